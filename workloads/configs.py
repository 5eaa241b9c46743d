"""The five benchmark workloads, transcribed into explicit parameters.

Shapes follow Llama-3-8B layers (hidden 4096, MLP 14336, 8 KV heads of 128
giving 1024-wide k/v projections).  The pages the method comes from run their
measurements on real models (Llama-3.1-8B and Llama-2-7B through a serving
benchmark, see "[Hardware][TPU][V1] Better tpu multilora compilation",
benchmark thread, and "[LoRA] LoRA cuda graph specialization", Test Result);
these synthetic batches of the same layer shapes stand in for them.

Reading of the distribution notation: in "N(0, s)" the second argument is the
variance, so N(0, 1/D) has standard deviation 1/sqrt(D).  Where a workload
does not state a scale it is 1.0; where it does not state the activation
distribution it is N(0, 1); where it states no seed it uses seed 0.
"""

# idx recipes:
#   ("iid_with_base", S)          idx uniform over {-1, 0, .., S-1}
#   ("uniform_then_base", S, n)   idx uniform over {0..S-1}, then exactly n
#                                 distinct tokens (drawn without replacement)
#                                 set to -1
#   ("contiguous", S, run)        request j owns tokens [j*run, (j+1)*run) and
#                                 slot j
#   ("zipf", S, s)                i.i.d. P(slot k) proportional to (k+1)^-s
#   ("all_base",)                 every token -1

CONFIGS = {
    "tiny_bgmv": dict(
        title="Tiny BGMV: T=64, D=256, out=256, r=8, 4 slots, fp32",
        dtype="f32",
        T=64,
        S=4,
        r_max=8,
        ranks=None,
        idx=("iid_with_base", 4),
        scale=2.0,
        seed=0,
        problems=[
            dict(name="proj", D=256, out_sizes=(256,), x_var=0.02, A_var=0.02,
                 B_var=0.02, timed_expand=True),
        ],
    ),
    "decode_qproj": dict(
        title="Decode BGMV, Llama-3-8B q_proj: T=256, D=4096, out=4096, r=16, "
              "8 slots, fp16, 10% base tokens",
        dtype="f16",
        T=256,
        S=8,
        r_max=16,
        ranks=None,
        idx=("uniform_then_base", 8, 26),  # round(0.1 * 256) = 26
        scale=2.0,  # alpha / r = 32 / 16
        seed=0,
        problems=[
            dict(name="q_proj", D=4096, out_sizes=(4096,), x_var=1.0,
                 A_var=1.0 / 4096, B_var=0.01, timed_expand=True),
        ],
    ),
    "prefill_qkv": dict(
        title="Prefill SGMV, fused QKV: 16 requests x 512 tokens, D=4096, "
              "out slices (4096, 1024, 1024), r=64, 16 slots, bf16",
        dtype="bf16",
        T=8192,
        S=16,
        r_max=64,
        ranks=None,
        idx=("contiguous", 16, 512),
        scale=1.0,
        seed=0,
        problems=[
            dict(name="qkv_proj", D=4096, out_sizes=(4096, 1024, 1024),
                 x_var=1.0, A_var=0.02, B_var=0.02, timed_expand=True),
        ],
    ),
    "mixed_rank_mlp": dict(
        title="Mixed-rank MLP: T=1024 decode tokens, gate/up 4096 -> 2x14336 and "
              "down shrink 14336 -> r, 32 slots, ranks in {8,16,32,64} padded to "
              "64, 50% base tokens, bf16",
        dtype="bf16",
        T=1024,
        S=32,
        r_max=64,
        ranks=(8, 16, 32, 64),
        idx=("uniform_then_base", 32, 512),
        scale=1.0,
        seed=0,
        problems=[
            dict(name="gate_up_proj", D=4096, out_sizes=(14336, 14336),
                 x_var=1.0, A_var=0.02, B_var=0.02, timed_expand=True),
            # The down projection's expand (r -> 4096) is drawn so that it can be
            # checked, but only its shrink is part of the timed step.
            dict(name="down_proj", D=14336, out_sizes=(4096,), x_var=1.0,
                 A_var=0.02, B_var=0.02, timed_expand=False),
        ],
    ),
    "zipf_many": dict(
        title="Many adapters, skewed: T=4096, D=4096, out=4096, r=32, 128 slots "
              "with Zipf(1.1) popularity, fp16",
        dtype="f16",
        T=4096,
        S=128,
        r_max=32,
        ranks=None,
        idx=("zipf", 128, 1.1),
        scale=1.0,
        seed=0,
        problems=[
            dict(name="proj", D=4096, out_sizes=(4096,), x_var=1.0,
                 A_var=1.0 / 4096, B_var=0.01, timed_expand=True),
        ],
    ),
    "zipf_many_noop": dict(
        title="The all-base batch of the same shape as zipf_many: every token -1",
        dtype="f16",
        T=4096,
        S=128,
        r_max=32,
        ranks=None,
        idx=("all_base",),
        scale=1.0,
        seed=0,
        problems=[
            dict(name="proj", D=4096, out_sizes=(4096,), x_var=1.0,
                 A_var=1.0 / 4096, B_var=0.01, timed_expand=True),
        ],
    ),
}

# Benchmark order; the first entry is the small case every CPU test can afford.
CONFIG_ORDER = ["tiny_bgmv", "decode_qproj", "prefill_qkv", "mixed_rank_mlp",
                "zipf_many", "zipf_many_noop"]


def describe(name):
    """One-line description of a workload with its sizes."""
    c = CONFIGS[name]
    return f"{name}: {c['title']}"
