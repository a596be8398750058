// The 32x32x16 matrix-core attention at head_dim 256 with 8 query heads per KV
// head (attention32.hip): launchers used by the entry points in attention.hip.
#pragma once

#include "common.h"
#include "engine.h"

namespace pi32 {

// Key splits of a prefill of B samples x Hkv KV heads over L tokens, and the
// workspace bytes of their partials (0 for one split).
int prefill_splits(int B, int Hkv, int L);
size_t prefill_split_bytes(int B, int Hkv, int L, int splits);
// Prefill (q [B, L, Hq, d], k / v [B, L, Hkv, d], o like q; Hq = 8 * Hkv, d = 256):
// splits the keys when split_ws holds prefill_split_bytes for the chosen split.
pi_status prefill(const void* q, const void* k, const void* v, void* o, int B, int L, int Hq, int Hkv, float scale,
                  const pi_mask* m, float rope_base, float* lse, void* split_ws, size_t split_avail, hipStream_t s);

// Key splits of a cached decode of B samples x S suffix tokens over `len` cache
// slots, and the workspace bytes of their partials.
int decode_splits(int B, int S, int len);
size_t decode_split_bytes(int B, int S, int splits);
// Cached decode of one layer (ckl / cvl: that layer's cache slices; Hq = 8, d = 256);
// q_s / o_s row-major [B, S, 8, 256], or with `tiled` the operand tile layout
// (see pi::decode_layer).
pi_status decode(const pi_kv_cache* cache, const __bf16* ckl, const __bf16* cvl, const void* q_s, const void* k_s,
                 const void* v_s, const uint8_t* suffix_ar, int B, int S, float scale, float rope_base, void* o_s,
                 bool tiled, void* split_ws, size_t split_avail, hipStream_t s);

// dK, dV of the attention backward (shapes as dq below; dk, dv [B, L, 1, 256]):
// dk = scale * sum over visible rows of dS q, dv = sum of P dO.
pi_status dkdv(const void* q, const void* k, const void* v, const void* dout, const float* lse2, const float* dr,
               void* dk, void* dv, int B, int L, float scale, const pi_mask* m, hipStream_t s);

// dQ of the attention backward (Hq = 8, Hkv = 1, d = 256; q, dout, dq [B, L, 8, 256],
// k, v [B, L, 1, 256], lse2 / dr [B, L, 8]: the rows' log-sum-exp in base 2 and
// dO . O): dq = scale * sum over visible keys of P (dP - Dr) k.
pi_status dq(const void* q, const void* k, const void* v, const void* dout, const float* lse2, const float* dr, void* dq,
             int B, int L, float scale, const pi_mask* m, hipStream_t s);

}  // namespace pi32
