"""Workload shapes and seeded synthetic inputs (shared by the oracle tests, the
GPU parity tests and the benchmark; contains none of the verification arithmetic)."""
from .configs import (BLOCK_SIZE, KV_BF16, KV_FP8, Workload, NAMED, MINI, EDGE, SWEEP_D,
                      TINY, LLAMA3_8B, LLAMA31_70B, FP8_LONG, tile_sweep, all_workloads)
from .generate import (AttnInputs, AcceptPlan, make_attn_inputs, make_accept_plan,
                       drafts_from_target, f32_to_bf16_bits, f32_to_e4m3_bits, seed_streams,
                       SampledAcceptInputs, make_sampled_accept_inputs, AppendInputs,
                       make_append_inputs, make_draft_logits, TreePlan,
                       make_tree_plan, tree_tokens_from_target, split_path_lengths)
