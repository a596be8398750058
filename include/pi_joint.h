/*
 * pi_joint.h -- C ABI of the MI355X (gfx950) block prefix-LM joint-attention path.
 *
 * The operations follow the π0 / π0.5 action-generation path described in
 *   [P1] "VLA 代码精读 — OpenPI & StarVLA", Part 1 (§1.2 mask and Euler sampling,
 *        §1.5 joint forward, §1.6 sample_actions with a prefix KV cache);
 *   [P3] "π0.5 vs MM-DiT joint attention" (hebangwen): one shared KV pool and one
 *        softmax, 8 query heads / 1 KV head / head_dim 256, the π0.5 three-block
 *        permission table, the cumsum block rule;
 *   [P4] "Pi0-FAST 模型架构", §2.3 (mask AND padding), §4.1 (KV-cache decode).
 *
 * Conventions for every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, contiguous, in the
 *     layouts stated below, 16-byte aligned.  bf16 tensors are passed as void*.
 *     Host-pointer arguments are marked (host).
 *   - The library never allocates, frees or synchronises inside these calls.
 *     Scratch memory is passed in as a workspace whose size is queried first.
 *   - Arguments are validated on the host before anything is launched; a bad
 *     argument returns PI_ERR_INVALID_ARG, an unsupported shape
 *     PI_ERR_UNSUPPORTED, a too-small workspace PI_ERR_WORKSPACE, and nothing
 *     is launched.  A launch failure returns PI_ERR_HIP.  Faults inside a kernel
 *     surface at the caller's next synchronisation.
 *   - `stream` is a hipStream_t (NULL = the default stream).  All work of one call
 *     is ordered on that stream.  There is no global mutable state; concurrent
 *     calls on different streams need distinct output buffers and workspaces.
 *   - pi_last_error() returns a description of the most recent failure on the
 *     calling thread.
 */
#ifndef PI_JOINT_H
#define PI_JOINT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pi_status {
  PI_OK = 0,
  PI_ERR_INVALID_ARG = -1,
  PI_ERR_UNSUPPORTED = -2,
  PI_ERR_WORKSPACE = -3,
  PI_ERR_HIP = -4
} pi_status;

typedef void* pi_stream; /* hipStream_t */

/* Segment tags used by the forbidden-pair rule ([P3] permission table). */
#define PI_SEG_PREFIX 0
#define PI_SEG_FAST 1
#define PI_SEG_EXPERT 2
/* Bit (4*query_seg + key_seg) of a forbid mask: that query segment may not read that key segment. */
#define PI_FORBID(qs, ks) (1u << (4u * (qs) + (ks)))

/* Granularity of the mask's tile table: 16 query tokens x 32 key tokens. */
#define PI_MASK_TILE_Q 16
#define PI_MASK_TILE_K 32
/* Tile classes stored in pi_mask.tiles. */
#define PI_TILE_EMPTY 0   /* no (query, key) pair of the tile is visible: skipped */
#define PI_TILE_PARTIAL 1 /* some pairs visible: evaluate the rule per pair */
#define PI_TILE_FULL 2    /* every pair visible: no per-pair test */

/*
 * Block prefix-LM mask in compact form ([P1] §1.2/§1.5, [P3] cumsum rule and
 * permission table, [P4] §2.3).  Key j is visible from query i of sample b iff
 *     bid[j] <= bid[i]  and  valid[b,i]  and  valid[b,j]
 *     and bit (4*seg[i] + seg[j]) of forbid_bits is clear,
 * with bid = inclusive cumsum of ar.  No N x N mask is stored.  All pointers are
 * device pointers into the workspace given to pi_mask_build; the struct itself
 * is host memory filled by pi_mask_build.
 *   bid   int32 [N]          inclusive cumsum of ar
 *   pos   int32 [B, N]       cumsum(valid) - 1 (token positions, [P1] §1.5)
 *   tok   uint32 [B, N]      packed per-token word: bit0 valid, bits1-2 seg, bits3.. bid
 *   tiles uint8 [B, n_qt, n_kt]  PI_TILE_* class of each 16x32 (query, key) tile
 */
typedef struct pi_mask {
  int32_t B, N;
  int32_t n_qt, n_kt;
  uint32_t forbid_bits;
  int32_t* bid;
  int32_t* pos;
  uint32_t* tok;
  uint8_t* tiles;
} pi_mask;

/* Workspace bytes pi_mask_build needs for B samples of N tokens. */
size_t pi_mask_workspace_bytes(int B, int N);

/*
 * Build the compact mask.  input_mask uint8 [B,N] (nonzero = valid token),
 * ar uint8 [N] (nonzero = the token opens a new block; shared by the batch),
 * seg uint8 [N] or NULL (all PI_SEG_PREFIX; only the low two bits are used),
 * forbid_bits as PI_FORBID().  1 <= B <= 65535, 1 <= N <= 1<<20.
 * Integer results are exact.
 */
pi_status pi_mask_build(const uint8_t* input_mask, const uint8_t* ar, const uint8_t* seg,
                        uint32_t forbid_bits, int B, int N, void* workspace,
                        size_t workspace_bytes, pi_mask* out, pi_stream stream);

/* Test aid: expand the compact mask into dense uint8 [B,N,N] (1 = visible). */
pi_status pi_mask_materialize(const pi_mask* mask, uint8_t* dense, pi_stream stream);

/*
 * Joint-attention prefill over one shared KV pool ([P3] first section; [P1] §1.5):
 *   O[b,i,h,:] = sum_j softmax_j(scale * q[b,i,h,:].k[b,j,g,:]) v[b,j,g,:]
 * over the keys j visible from i under `mask`, g = floor(h*Hkv/Hq); one softmax
 * per (b, i, h).  Masked keys are excluded by selection: a masked score never
 * enters the maximum or the sum and its weight is exactly 0.  What that
 * guarantees for the values a masked key holds:
 *   - K of a masked key, and K and V of a padded (invalid) key, never reach an
 *     output, whatever they hold (NaN and inf included): padded keys are
 *     staged as zeros;
 *   - a finite V of a valid key that is masked for some rows cannot change
 *     those rows' outputs (bit-exact);
 *   - NOT guaranteed: an inf or NaN in the V of a valid key that some rows of
 *     the same 16-query x 32-key tile may read and others may not (say a FAST
 *     token's V, which π0.5's expert rows may not read) enters the masked
 *     rows' product with weight 0 and gives 0 * inf = NaN there.
 * A query with no visible key gets O = 0.
 *   q  bf16 [B, L, Hq, d]    k, v  bf16 [B, L, Hkv, d]    o  bf16 [B, L, Hq, d]
 *   mask built for the same B and N = L.  scale > 0 (usually 1/sqrt(d)).
 * Supported heads: (Hq, Hkv, d) = (8, 1, 256) and (Hq, Hkv, d) with Hq == Hkv and
 * d = 64.  bf16 matrix-core products with fp32 accumulation.
 * rope_base: 0 = no rotary embedding; > 1 = q and k are rotated at the mask's
 * positions (pi_mask.pos) before the scores, as pi_rope_apply does (k into the
 * workspace, q in registers; the inputs are left untouched).
 * lse (device, optional, fp32 [B, L, Hq]): when non-NULL, each row's natural-log
 * log-sum-exp of its visible scaled scores, log sum_j exp(scale q.k_j) (-inf for
 * a row with no visible key), the statistic pi_joint_attn_backward takes.
 * If `cache` is non-NULL, K/V rows of tokens [0, cache->len) are also copied to
 * cache layer `layer` (cache->B == B, cache->len <= L); with the rotary
 * embedding the cache receives the rotated keys.
 * workspace (device, 256-byte aligned): pi_prefill_workspace_bytes(B, L, Hq, Hkv, d)
 * bytes cover every use.  Required with rope_base > 0 (PI_ERR_WORKSPACE without);
 * otherwise optional: with it a batch too small to fill the chip splits each
 * query block's keys over several workgroups and merges the partial softmaxes
 * (same result up to rounding order), without it the call runs unsplit.  Calls
 * that share a workspace must not overlap.
 */
typedef struct pi_kv_cache pi_kv_cache;
size_t pi_prefill_workspace_bytes(int B, int L, int Hq, int Hkv, int d);
pi_status pi_joint_attn_prefill(const void* q, const void* k, const void* v, int B, int L, int Hq,
                                int Hkv, int d, float scale, float rope_base, const pi_mask* mask,
                                void* o, float* lse, const pi_kv_cache* cache, int layer,
                                void* workspace, size_t workspace_bytes, pi_stream stream);

/*
 * Backward of the joint-attention prefill ([P1] §1.5: training runs the same
 * joint forward under the block mask and differentiates the loss through it).
 * Given the upstream gradient dO = dLoss/dO, per query row (b, i, h) with visible
 * keys j (the one KV head):
 *   P_j = exp(scale q.k_j - lse),  dP_j = dO.v_j,  Dr = dO.O,  dS_j = P_j (dP_j - Dr)
 *   dq[b,i,h] = scale sum_j dS_j k_j;   dk[b,j] += scale dS_j q[b,i,h];   dv[b,j] += P_j dO[b,i,h]
 * (sums over every row that sees key j).  Masked pairs contribute exactly
 * nothing; a row with no visible key gets dq = 0, and a key no row sees gets
 * dk = dv = 0.  Q/dO of padded tokens and K/V of padded keys may hold anything
 * (staged as zeros).  As in the forward, an inf or NaN in the K or V of a valid
 * key that only some rows of a tile may read reaches the other rows' dq as NaN
 * (its weight is 0, its dP is not finite).
 *   q, o, dout, dq  bf16 [B, L, Hq, d]    k, v, dk, dv  bf16 [B, L, Hkv, d]
 *   lse  fp32 [B, L, Hq]: the forward's log-sum-exp (pi_joint_attn_prefill's lse
 *        output for the same q, k, mask, scale and rope_base); o: its output.
 *   mask built for the same B and N = L; scale as in the forward.
 * Supported: (Hq, Hkv, d) = (8, 1, 256).  rope_base: 0, or the forward's rotary
 * base (> 1): q and k are then the unrotated inputs the forward rotated at the
 * mask's positions, and dq, dk are the gradients of those (the rotated
 * gradients turned back by the negated positions, R(p)^T = R(-p); one more bf16
 * rounding).  bf16 matrix-core products with fp32 accumulation; P and dS are
 * rounded to bf16 as operands, the gradients to bf16 on output.  Outputs must
 * not overlap the inputs.  Three kernels on `stream` (row statistics, dk/dv
 * key-major, dq query-major); no atomics, so results are deterministic.
 * workspace (device, 256-byte aligned, required):
 * pi_attn_backward_workspace_bytes(B, L, Hq, Hkv, d, rope_base) bytes (0 = unsupported).
 */
size_t pi_attn_backward_workspace_bytes(int B, int L, int Hq, int Hkv, int d, float rope_base);
pi_status pi_joint_attn_backward(const void* q, const void* k, const void* v, const void* o,
                                 const void* dout, const float* lse, int B, int L, int Hq, int Hkv,
                                 int d, float scale, float rope_base, const pi_mask* mask, void* dq,
                                 void* dk, void* dv, void* workspace, size_t workspace_bytes,
                                 pi_stream stream);

/*
 * One π0.5 joint transformer layer around the joint attention ([P3] first
 * section: each stream has its own norm, QKV projection, output projection and
 * FFN, the streams share one concatenated KV pool and one softmax; [P1] §1.4:
 * the π0.5 action expert normalises with an adaptive RMS norm conditioned on the
 * flow time, §2.7 the adaptive norm's shift / scale form).  Per stream, with
 * n(h) = h / sqrt(mean(h^2) + 1e-6) over the width and r() rounding to bf16:
 *   a = r(n(h) * norm1)  or  r(n(h) * (1 + scale1) + shift1),  [shift1 | scale1] = r(silu(cond)) mod1^T
 *   q | k | v = r(a w_qkv^T)            (8 query heads, 1 KV head, d = 256)
 *   o = r(joint attention over the concatenated [prefix | expert] tokens under mask)
 *   h += o[stream rows] w_o^T
 *   b = r(n(h) * norm2)  or  the adaptive form with mod2
 *   h += r(gelu(b w_up^T)) w_down^T     (gelu(x) = x Phi(x))
 * The norm, FFN and rounding details are readings of the pages.
 *   h_p fp32 [B, Np, prefix->width], h_e fp32 [B, Ne, expert->width], updated in place
 *   cond fp32 [B, width of the adaptive stream] (NULL if neither stream is adaptive)
 *   mask built for B and N = Np + Ne, the prefix stream's tokens first
 * Weights (device, bf16 row-major, out x in): w_qkv [2560, W], w_o [W, 2048],
 * w_up [ffn, W], w_down [W, ffn]; norm1 / norm2 fp32 [W] for a plain norm, or
 * mod1 / mod2 bf16 [2W, W] for an adaptive one (exactly one of the two pairs;
 * at most one adaptive stream).  W and ffn multiples of 256, W <= 4096,
 * ffn <= 65536; every activation below 2 GiB (else PI_ERR_UNSUPPORTED).  Every
 * product runs on the matrix cores with fp32 accumulation.
 * workspace (device, 256-byte aligned, required): pi_joint_layer_workspace_bytes
 * (0 = unsupported streams).  Calls sharing a workspace must not overlap.
 */
typedef struct pi_layer_stream {
  int32_t width, ffn;
  const void* w_qkv;
  const void* w_o;
  const void* w_up;
  const void* w_down;
  const float* norm1;
  const float* norm2;
  const void* mod1;
  const void* mod2;
} pi_layer_stream;
size_t pi_joint_layer_workspace_bytes(const pi_layer_stream* prefix, const pi_layer_stream* expert, int B,
                                      int Np, int Ne);
pi_status pi_joint_layer_forward(const pi_layer_stream* prefix, const pi_layer_stream* expert, float* h_p,
                                 float* h_e, const float* cond, int B, int Np, int Ne, float scale,
                                 const pi_mask* mask, void* workspace, size_t workspace_bytes,
                                 pi_stream stream);

/*
 * The prefix stream's half of the same layer alone, writing the layer's K/V into
 * the cache ([P1] §1.6: at inference the prefix is run once and its K/V cached;
 * under the π0.5 mask no prefix token sees an expert token, so the prefix rows of
 * pi_joint_layer_forward do not depend on the expert and this is that layer with
 * Ne = 0).  h_p fp32 [B, Np, width] updated in place; mask built for B and N = Np
 * (the prefix's own block mask); the cache (cache->B == B, cache->len == Np) gets
 * the prefix tokens' K/V in slots [0, Np) of layer `layer`; the caller sets the
 * cache's prefix_mask to the prefix's input mask.  cond as pi_joint_layer_forward
 * (NULL for a plain-norm stream).  workspace: pi_prefix_layer_workspace_bytes.
 */
size_t pi_prefix_layer_workspace_bytes(const pi_layer_stream* prefix, int B, int Np);
pi_status pi_prefix_layer_forward(const pi_layer_stream* prefix, float* h_p, const float* cond, int B,
                                  int Np, float scale, const pi_mask* mask, const pi_kv_cache* cache,
                                  int layer, void* workspace, size_t workspace_bytes, pi_stream stream);

/*
 * The expert stream's half of the same layer in the cached form ([P1] §1.6: at
 * inference the prefix is computed once and each Euler step runs only the
 * suffix against the cache): the S expert tokens h_e fp32 [B, S, W] (updated in
 * place) take norm 1 and their fused QKV as in pi_joint_layer_forward, attend
 * to the valid slots of cache layer `layer` plus their own K/V under suffix_ar
 * (pi_suffix_decode_step), then take the output projection, norm 2 and FFN.
 * The cache holds the prefix stream's K/V of that layer.  Same stream
 * weights and cond as above; S and the cache as pi_suffix_decode_step supports.
 * workspace (device, 256-byte aligned, required):
 * pi_expert_layer_decode_workspace_bytes(expert, B, S, cache->len).
 */
size_t pi_expert_layer_decode_workspace_bytes(const pi_layer_stream* expert, int B, int S, int len);
pi_status pi_expert_layer_decode(const pi_layer_stream* expert, const pi_kv_cache* cache, int layer,
                                 float* h_e, const float* cond, const uint8_t* suffix_ar, int B, int S,
                                 float scale, void* workspace, size_t workspace_bytes, pi_stream stream);

/*
 * Per-layer prefix KV cache ([P1] §1.6; [P4] §4.1).  Device memory owned by the caller.
 *   k, v         bf16 [layers, B, capacity, Hkv, d]
 *   prefix_mask  uint8 [B, capacity]: nonzero = slot holds a valid prefix token
 *   len          slots in use (the prefix length P), <= capacity
 * When capacity == L the per-layer slices k + layer*B*capacity*Hkv*d are laid out
 * exactly as the prefill's k/v inputs, so a prefix-only prefill can read them in place.
 */
struct pi_kv_cache {
  void* k;
  void* v;
  const uint8_t* prefix_mask;
  int32_t layers, B, capacity, Hkv, d;
  int32_t len;
};

/*
 * Cached suffix decode for one layer ([P1] §1.6): the S suffix queries attend to
 * the valid prefix slots of cache layer `layer` plus the suffix keys allowed by
 * the suffix's own block rule (suffix key j visible from suffix query i iff
 * cumsum(suffix_ar)[j] <= cumsum(suffix_ar)[i]); all suffix tokens are valid.
 *   q_s  bf16 [B, S, Hq, d]   k_s, v_s  bf16 [B, S, Hkv, d]   o_s  bf16 [B, S, Hq, d]
 *   suffix_ar  uint8 [S] (device)
 * Supported: Hq = 8, Hkv = 1, d = 256, 1 <= S <= 128.  Each cached K/V tile is
 * read from HBM once per sample and shared by all 8 query heads.
 * rope_base: 0 = no rotary embedding; > 1 = q_s and k_s are rotated with token t
 * of sample b at position (valid slots of prefix_mask[b]) + t ([P1] §1.6), and
 * the cache is taken to hold keys already rotated (as a prefill with the same
 * rope_base writes them).
 * workspace (device, 256-byte aligned): pi_decode_workspace_bytes(B, S, Hq,
 * cache->len) bytes cover every use.  Required with rope_base > 0; otherwise
 * optional: with it a small batch splits each sample's keys over several
 * workgroups and merges the partial softmaxes, without it the call runs unsplit
 * (same result up to rounding).
 * Masked keys as in pi_joint_attn_prefill: padded cache slots may hold anything,
 * NaN included (they are staged as zeros, or, in the few-sample kernel, loaded,
 * their V rows zeroed and their scores masked); an inf or NaN in the V of a
 * suffix key that only some suffix rows may read can reach the others as NaN.
 */
size_t pi_decode_workspace_bytes(int B, int S, int Hq, int len);
pi_status pi_suffix_decode_step(const pi_kv_cache* cache, int layer, const void* q_s,
                                const void* k_s, const void* v_s, const uint8_t* suffix_ar,
                                int B, int S, int Hq, float scale, float rope_base, void* o_s,
                                void* workspace, size_t workspace_bytes, pi_stream stream);

/*
 * Allocation-free variant of pi_suffix_decode_step, for callers that cannot
 * allocate device memory or pass a workspace: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.  Same arguments,
 * layouts and result as pi_suffix_decode_step minus the workspace.  Its scratch
 * (the rotated suffix keys under the rotary embedding, the key-split partials
 * of a small batch) is one file-scope device array of PI_NOALLOC_SCRATCH_BYTES
 * per GPU, held from the library's load until the process ends; the call
 * allocates and frees nothing.  The key split runs when its partials fit the
 * scratch, exactly as pi_suffix_decode_step with a workspace of that size
 * (bit-identical to it then); otherwise the call runs unsplit.  Returns
 * PI_ERR_UNSUPPORTED, launching nothing, when the rotated suffix keys alone
 * (B * S * 512 bytes, rope_base > 0) exceed the scratch.  Every call on one GPU
 * shares that GPU's scratch, which keeps the last call's contents (nothing in it
 * needs to start at zero): calls that overlap on one GPU (different streams,
 * threads) race and must be serialised by the caller.
 */
#define PI_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)
pi_status pi_suffix_decode_step_noalloc(const pi_kv_cache* cache, int layer, const void* q_s,
                                        const void* k_s, const void* v_s, const uint8_t* suffix_ar,
                                        int B, int S, int Hq, float scale, float rope_base, void* o_s,
                                        pi_stream stream);

/*
 * Single-token autoregressive decode ([P4] §4.1: after the prefill, every step
 * runs one new token against the cache, which then keeps its K/V).  A step is
 * pi_suffix_decode_step with S = 1 and suffix_ar = {1} (the token sees every
 * valid cache slot and itself; a one-wave workgroup per key split), followed by
 * pi_kv_cache_append of the token's k/v to every layer, after which the caller
 * raises cache->len by n_new.
 *
 * Append n_new tokens per sample to cache layer `layer` at slots
 * [len, len + n_new): k_new, v_new bf16 [B, n_new, Hkv, d]; their prefix_mask
 * bytes are set to 1 (the mask's const qualifier in pi_kv_cache only says the
 * attention calls read it).  With rope_base > 1 the keys are stored rotated,
 * token t at (valid slots among [0, len)) + t, as the decode rotates its query.
 * Requires len + n_new <= capacity; d a multiple of 16 up to 512.
 */
pi_status pi_kv_cache_append(const pi_kv_cache* cache, int layer, const void* k_new, const void* v_new,
                             int n_new, float rope_base, pi_stream stream);

/*
 * Rotary position embedding ([P1] §3.2: π0 keeps its LLM's rotary embedding;
 * positions per §1.5 / §1.6, e.g. pi_mask.pos).  For each token t of each sample
 * and each head, with p = pos[b*L + t] and i < d/2:
 *   y[i]       = x[i] cos(a) - x[i + d/2] sin(a)
 *   y[i + d/2] = x[i + d/2] cos(a) + x[i] sin(a),   a = p * base^(-2i/d)
 * (the rotate-half arrangement; the pages name the method, not the formula).
 *   x, y  bf16 [B, L, H, d] (y may equal x)   pos  int32 [B, L] (device)
 * d a multiple of 16 up to 512, base > 1 (usually 10000).  fp32 arithmetic with
 * the angle reduced in fp64; bf16 results.
 */
pi_status pi_rope_apply(const void* x, void* y, int B, int L, int H, int d, const int32_t* pos,
                        float base, pi_stream stream);

/* Euler update x <- x + dt * v over n fp32 elements ([P1] §1.2). */
pi_status pi_euler_update(float* x, const float* v, float dt, int64_t n, pi_stream stream);

/*
 * Stand-in velocity net (random weights; the pages give no weights).  nn.Linear
 * layout [out, in]; matrices bf16, vectors fp32.  W = width, A = action_dim.
 *   w_state [W, A], b_state [W]        state token  = r(state) W_state^T + b_state
 *   w_in    [W, A], b_in [W], w_time [W]  action tokens = r(x) W_in^T + b_in + t*w_time
 *   w_q [Hq*d, W], w_k, w_v [Hkv*d, W], w_o [W, Hq*d]
 *       per cache layer l: a = r(h); q,k,v = r(a W^T / rms(a)); o = r(decode_l(q,k,v));
 *                          h += o W_o^T
 *   w_out [A, W], b_out [A]            velocity = a[:,1:] W_out^T / rms(a[:,1:]) + b_out,
 *                                      a = r(h) after the last layer
 * r() rounds to bf16; products accumulate in fp32; h is fp32.  rms(a) =
 * sqrt(mean(a^2) + 1e-6) over the width is the per-stream RMS norm ahead of the
 * projections ([P3] first section), a per-row scalar applied to the product.
 * The same weights serve every cache layer.
 */
typedef struct pi_velocity_net {
  int32_t width, action_dim, Hq, Hkv, d;
  const void* w_state;
  const float* b_state;
  const void* w_in;
  const float* b_in;
  const float* w_time;
  const void* w_q;
  const void* w_k;
  const void* w_v;
  const void* w_o;
  const void* w_out;
  const float* b_out;
} pi_velocity_net;

/* Workspace bytes for pi_velocity_eval / pi_flow_sample with B samples of H actions. */
size_t pi_flow_workspace_bytes(const pi_velocity_net* net, int B, int H);

/*
 * One evaluation of the stand-in velocity net at time t (the suffix forward of
 * one denoising step, [P1] §1.6).  x fp32 [B,H,A]; state fp32 [B,A];
 * suffix_ar uint8 [H+1] (device; state token first); vel fp32 [B,H,A].
 * Uses cache layers [0, cache->layers).  Width W must be a multiple of 64,
 * A <= 64, H + 1 <= 128.  The workspace also holds the weights repacked into the
 * matrix-core operand layout, redone at the start of every call (so weights may
 * change between calls).
 */
pi_status pi_velocity_eval(const pi_velocity_net* net, const pi_kv_cache* cache,
                           const uint8_t* suffix_ar, const float* state, const float* x, float t,
                           float* vel, int B, int H, int A, void* workspace,
                           size_t workspace_bytes, pi_stream stream);

/*
 * Euler flow-matching sampler ([P1] §1.2, §1.6): x holds the noise on entry and
 * the sampled actions on exit; dt = -1/num_steps; step k evaluates the velocity
 * at t_k = 1 + k*dt and sets x <- x + dt*v.
 *   net != NULL: v = the stand-in velocity net (pi_velocity_eval); the output
 *                projection and the Euler update are fused.
 *   net == NULL: v = v_const fp32 [B,H,A] (closed-form check: x_N = noise - v).
 * x fp32 [B,H,A] in place.  num_steps >= 1.
 */
pi_status pi_flow_sample(const pi_velocity_net* net, const pi_kv_cache* cache,
                         const uint8_t* suffix_ar, const float* state, const float* v_const,
                         float* x, int B, int H, int A, int num_steps, void* workspace,
                         size_t workspace_bytes, pi_stream stream);

/*
 * π0.5's action expert at its true shape as the velocity net of the Euler
 * sampler ([P1] §1.4: the noisy actions are projected to the expert's width,
 * the flow time passes through the expert's own two-layer MLP whose output
 * conditions the adaptive RMS norms, and the expert's outputs are projected back
 * to the action dim; §1.6: the prefix is cached once and each step runs only the
 * expert tokens against it; §1.2: the sampler).  Per evaluation at time t, with
 * r() rounding to bf16 and W the width:
 *   emb[j] = sin(2 pi t / p_j), emb[W/2 + j] = cos(2 pi t / p_j),  p_j = 4e-3 * 1000^(j / (W/2 - 1))
 *   c = r(silu(r(emb) w_t1^T + b_t1)) w_t2^T + b_t2           (the same for every sample)
 *   h = r(x) w_in^T + b_in                                     (the H action tokens)
 *   h = layer l in the cached form against cache layer l, l < layers (pi_expert_layer_decode, cond = c)
 *   v = r(n(h) * (1 + scale) + shift) w_out^T + b_out,  [shift | scale] = r(silu(c)) mod_f^T
 * The embedding, the MLP's activation and the final norm are readings of the
 * pages.  Attention scale 1/16 (head_dim 256).
 * Weights (device): w_in bf16 [W, A], w_t1 / w_t2 bf16 [W, W], mod_f bf16 [2W, W],
 * w_out bf16 [A, W]; biases fp32 b_in / b_t1 / b_t2 [W], b_out [A]; `layer` is a
 * host array of `layers` expert streams of width W with adaptive norms (mod1,
 * mod2).  W a multiple of 256 (<= 4096), 1 <= A <= 256, layers >= 1, the cache
 * with B samples and at least `layers` layers, H <= 128.
 */
typedef struct pi_expert_net {
  int32_t width, action_dim, layers;
  const void* w_in;
  const float* b_in;
  const void* w_t1;
  const float* b_t1;
  const void* w_t2;
  const float* b_t2;
  const pi_layer_stream* layer;
  const void* mod_f;
  const void* w_out;
  const float* b_out;
} pi_expert_net;

/* Workspace bytes of pi_expert_velocity_eval (num_steps = 1) and pi_expert_flow_sample
 * for B samples of H actions over a cache of `len` slots (0 = unsupported). */
size_t pi_expert_flow_workspace_bytes(const pi_expert_net* net, int B, int H, int len, int num_steps);

/* One evaluation at time t (the embedding is taken at (double)t): x fp32 [B,H,A],
 * vel fp32 [B,H,A]; suffix_ar uint8 [H] (device), the expert tokens' block
 * starts (π0.5: the first action opens the block). */
pi_status pi_expert_velocity_eval(const pi_expert_net* net, const pi_kv_cache* cache,
                                  const uint8_t* suffix_ar, const float* x, float t, float* vel,
                                  int B, int H, int A, void* workspace, size_t workspace_bytes,
                                  pi_stream stream);

/* The Euler sampler with this net: x holds the noise on entry and the actions on
 * exit; dt = -1/num_steps, step k at t_k = 1 + k*dt (computed in double); the
 * conditioning rows of all steps are computed once at the start; the output
 * projection and x <- x + dt*v are fused.  1 <= num_steps <= 1000. */
pi_status pi_expert_flow_sample(const pi_expert_net* net, const pi_kv_cache* cache,
                                const uint8_t* suffix_ar, float* x, int B, int H, int A,
                                int num_steps, void* workspace, size_t workspace_bytes,
                                pi_stream stream);

/* Text of a status code, and the last failure's description on this thread. */
const char* pi_status_string(pi_status status);
const char* pi_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PI_JOINT_H */
