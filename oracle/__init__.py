"""fp64 CPU oracle for block prefix-LM joint attention (π0 / π0.5).

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute this package; only the tests, the smoke entry point and the
benchmark's CPU-baseline leg use it.  It shares no code with the HIP path.

What it computes, in plain numpy float64 with an explicit [B, N, N] mask:

  mask.block_ids / mask.attn_mask / mask.positions / mask.decode_mask
      the cumsum block mask AND padding AND forbidden segment pairs, and the
      token positions ("VLA 代码精读 — OpenPI & StarVLA" §1.2, §1.5, §1.6;
      "π0.5 vs MM-DiT joint attention", three-block permission table;
      "Pi0-FAST 模型架构" §2.3).
  attention.joint_attention
      one softmax over the concatenated prefix+suffix KV pool with grouped
      query heads ("π0.5 vs MM-DiT joint attention", first section).
  attention.cached_decode
      suffix queries over cached prefix K/V plus their own K/V
      ("VLA 代码精读" §1.6).
  flow.euler_sample / flow.euler_update
      the Euler flow-matching sampler, t from 1 to 0 ("VLA 代码精读" §1.2, §1.6).
  attention_bwd.masked_attention_grads / attention_bwd.lse_rows
      the gradients of the masked attention from their definitions, and the
      rows' log-sum-exp (training differentiates the same joint forward,
      "VLA 代码精读" §1.5).
  rope.rope / rope.joint_attention_rope
      the rotary position embedding of Q and K at the mask's positions
      ("VLA 代码精读" §3.2, §1.5, §1.6; the formula is a reading).
  layer.joint_layer
      one π0.5 joint transformer layer around the joint attention: per-stream
      norm (plain RMS for the prefix, adaptive RMS for the expert), fused QKV,
      concatenated KV pool, one masked softmax, split, output projection and
      FFN per stream ("π0.5 vs MM-DiT joint attention", first section; "VLA
      代码精读" §1.4, §2.7; the norm, FFN and rounding details are readings).
  expert_flow.expert_velocity / expert_flow.expert_flow_sample
      π0.5's action expert at its true shape driving the Euler sampler: action
      in-projection, time embedding and time MLP conditioning the adaptive
      norms, the expert layers against the cache layer by layer, a final
      adaptive norm and the action out-projection ("VLA 代码精读" §1.2, §1.4,
      §1.6; the embedding, MLP activation and final norm are readings).
  flow.velocity_net / flow.embed_suffix / flow.rms
      the random-weight stand-in velocity network.  The pages give only its
      shapes; its definition is a reading, pinned against a float64 composition
      of library calls (F.linear, scaled_dot_product_attention, vector_norm),
      a hand-written closed form with the attention path zeroed, and the
      state token's place at row 0.

Readings of points the pages leave open are listed in each docstring.
"""
from . import bf16, mask, attention, attention_bwd, flow, layer, rope, expert_flow  # noqa: F401
