"""Layer configuration and the named synthetic workloads.

Field names follow the model arguments of the "gate-init" excerpt on
"DeepSeek-V3.2-Exp - Routing weights" and of the V4.1 MoE class on
"DeepSeek V4.1 - Add shared"; the struct mirrors ``moe_config`` in moe.h.
"""

from dataclasses import dataclass, field, replace

SCORE = {"softmax": 0, "sigmoid": 1, "sqrtsoftplus": 2}
ROUTE = {"learned": 0, "hash": 1, "ngram": 2}
DTYPE = {"f32": 0, "bf16": 1, "fp4": 2, "fp8": 3}   # fp8: E4M3 in 128x128 blocks (re-dequantised FP4)
LAYOUT = {"rows": 0, "tiled": 1}
ACT_QUANT = {"none": 0, "mxfp8": 1}


@dataclass(frozen=True)
class MoEConfig:
    dim: int
    n_routed_experts: int
    n_activated_experts: int
    moe_inter_dim: int
    n_expert_groups: int = 1
    n_limited_groups: int = 1
    n_shared_experts: int = 1
    score_func: str = "softmax"
    route_scale: float = 1.0
    renormalize: int = -1
    swiglu_limit: float = 0.0
    route_mode: str = "learned"
    vocab_size: int = 0
    act_dtype: str = "bf16"
    expert_dtype: str = "bf16"
    has_bias: bool = False
    weight_layout: str = "rows"   # expert matrices as given ("rows") or packed ("tiled")
    act_quant: str = "none"       # FP4 routed experts: "mxfp8" activations on the scaled MFMA

    @property
    def renorm(self):
        if self.renormalize < 0:
            return self.score_func != "softmax"
        return bool(self.renormalize)


@dataclass(frozen=True)
class Workload:
    """A layer config, a token count and the recipe of its synthetic inputs."""
    name: str
    cfg: MoEConfig
    T: int
    zipf_s: float = 1.1          # hash routing: token frequency p_i ~ i^-s
    bias_range: float = 0.01     # bias ~ U(-r, r) when cfg.has_bias
    x_scale: float = 1.0         # x ~ N(0, x_scale^2)
    seed: int = 0
    x_rows: int = 0              # draw x with this many rows, keep the first T
    seq_len: int = 0             # 2-gram hash: tokens per sequence (0: one sequence)
    fp8_weights: bool = False    # FP4 layer run on its FP8 re-dequantisation (moe_redequant_fp8)
    description: str = ""


# The five layer workloads (the small tiny-fp32 one is cheap enough for the
# oracle at full size; the others are sampled by the parity tests).
TINY_FP32 = Workload(
    "tiny_fp32",
    MoEConfig(dim=128, n_routed_experts=16, n_activated_experts=2, moe_inter_dim=64,
              score_func="softmax", route_scale=1.0, act_dtype="f32", expert_dtype="f32"),
    T=64, description="T=64, d=128, 16 experts top-2, softmax, fp32")

HASH_BF16 = Workload(
    "hash_bf16",
    MoEConfig(dim=2048, n_routed_experts=64, n_activated_experts=4, moe_inter_dim=1024,
              route_mode="hash", vocab_size=32768, route_scale=1.0),
    T=4096, description="hash routing, m=32768 Zipf(1.1), 64 experts top-4, d=2048, I=1024, bf16")

V3_PREFILL = Workload(
    "v3_prefill",
    MoEConfig(dim=7168, n_routed_experts=256, n_activated_experts=8, moe_inter_dim=2048,
              n_expert_groups=8, n_limited_groups=4, score_func="sigmoid", route_scale=2.5,
              has_bias=True),
    T=4096, description="DeepSeek-V3 shape prefill, T=4096, d=7168, 256 experts (8 groups, keep 4) top-8")

V3_DECODE = replace(V3_PREFILL, name="v3_decode", T=64, x_rows=4096,
                    description="DeepSeek-V3 shape decode, T=64 (64 sequences x 1 position)")

V41_FLASH_FP4 = Workload(
    "v41_flash_fp4",
    MoEConfig(dim=5120, n_routed_experts=384, n_activated_experts=8, moe_inter_dim=1536,
              score_func="sqrtsoftplus", route_scale=1.0, swiglu_limit=10.0,
              expert_dtype="fp4", has_bias=True),
    T=8192, description="V4.1-Flash shape, T=8192, d=5120, 384 experts top-8, sqrt(softplus), "
                        "FP4 e2m1 + e8m0/32 routed experts, clamp 10")

NGRAM_BF16 = Workload(
    "ngram_bf16",
    replace(HASH_BF16.cfg, route_mode="ngram"),
    T=4096, seq_len=512,
    description="2-gram hash routing (previous id, id) -> (a*q_j + b) mod 64, 8 sequences of 512 "
                "Zipf(1.1) ids, d=2048, I=1024, bf16")

V41_FLASH_FP4_MX = replace(
    V41_FLASH_FP4, name="v41_flash_fp4_mx", cfg=replace(V41_FLASH_FP4.cfg, act_quant="mxfp8"),
    description="V4.1-Flash shape with the routed FP4 experts on MXFP8 activations "
                "(E4M3 + E8M0/32) and the scaled MFMA")

V41_FLASH_FP8 = replace(
    V41_FLASH_FP4_MX, name="v41_flash_fp8", fp8_weights=True,
    description="V4.1-Flash shape with the FP4 routed experts re-dequantised to FP8 E4M3 in "
                "128x128 blocks, on MXFP8 activations (FP8 x FP8 scaled MFMA)")

FULL_WORKLOADS = {w.name: w for w in (TINY_FP32, HASH_BF16, V3_PREFILL, V3_DECODE, V41_FLASH_FP4,
                                      NGRAM_BF16, V41_FLASH_FP4_MX, V41_FLASH_FP8)}

# Reduced versions: the same structure at sizes the oracle finishes in
# seconds while still spanning several GEMM tiles, slabs and a ragged tail.
SMALL_WORKLOADS = {
    "tiny_fp32": TINY_FP32,
    "ngram_small": Workload(
        "ngram_small",
        replace(HASH_BF16.cfg, dim=256, moe_inter_dim=128, n_routed_experts=16, vocab_size=2048,
                route_mode="ngram"),
        T=301, seq_len=64),
    "hash_small": Workload(
        "hash_small",
        replace(HASH_BF16.cfg, dim=256, moe_inter_dim=128, n_routed_experts=16, vocab_size=2048),
        T=301),
    "v3_small": Workload(
        "v3_small",
        replace(V3_PREFILL.cfg, dim=512, moe_inter_dim=256, n_routed_experts=64),
        T=203),
    "v3_decode_small": Workload(
        "v3_decode_small",
        replace(V3_PREFILL.cfg, dim=512, moe_inter_dim=256, n_routed_experts=64),
        T=13, x_rows=203),
    "fp4_small": Workload(
        "fp4_small",
        replace(V41_FLASH_FP4.cfg, dim=256, moe_inter_dim=128, n_routed_experts=48),
        T=157),
    "fp4_odd_widths": Workload(
        "fp4_odd_widths",
        replace(V41_FLASH_FP4.cfg, dim=320, moe_inter_dim=192, n_routed_experts=48),
        T=77),
    "fp4_mx_small": Workload(
        "fp4_mx_small",
        replace(V41_FLASH_FP4.cfg, dim=256, moe_inter_dim=128, n_routed_experts=48,
                act_quant="mxfp8"),
        T=157, description="FP4 experts on MXFP8 activations (scaled MFMA)"),
    "fp4_mx_decode": Workload(
        "fp4_mx_decode",
        replace(V41_FLASH_FP4.cfg, dim=256, moe_inter_dim=256, n_routed_experts=48,
                act_quant="mxfp8"),
        T=9, description="MXFP8 activations, decode batch: one-row-block tiles"),
    "fp4_mx_decode_narrow": Workload(
        "fp4_mx_decode_narrow",
        replace(V41_FLASH_FP4.cfg, dim=256, moe_inter_dim=384, n_routed_experts=48,
                act_quant="mxfp8"),
        T=9, description="MXFP8 activations, decode batch, a gate|up width that is a "
                         "multiple of 128 but not of 256 (4-wave decode kernel)"),
    "fp4_mx_clamp": Workload(
        "fp4_mx_clamp",
        replace(V41_FLASH_FP4.cfg, dim=384, moe_inter_dim=256, n_routed_experts=24,
                act_quant="mxfp8"),
        T=300, x_scale=20.0, description="MXFP8 activations with the clamp firing; 3 k-stages"),
    "fp8_mx_small": Workload(
        "fp8_mx_small",
        replace(V41_FLASH_FP4.cfg, dim=256, moe_inter_dim=128, n_routed_experts=48,
                act_quant="mxfp8"),
        T=157, fp8_weights=True,
        description="FP4 experts re-dequantised to FP8 (128x128 blocks) on MXFP8 activations"),
    "fp8_mx_decode": Workload(
        "fp8_mx_decode",
        replace(V41_FLASH_FP4.cfg, dim=256, moe_inter_dim=256, n_routed_experts=48,
                act_quant="mxfp8"),
        T=9, fp8_weights=True, description="FP8 weights, decode batch (run as 4-block tiles)"),
    "fp8_mx_clamp": Workload(
        "fp8_mx_clamp",
        replace(V41_FLASH_FP4.cfg, dim=384, moe_inter_dim=256, n_routed_experts=24,
                act_quant="mxfp8"),
        T=300, x_scale=20.0, fp8_weights=True,
        description="FP8 weights, clamp firing, 3 k-stages, two column slabs"),
    "fp4_clamp_small": Workload(
        "fp4_clamp_small",
        replace(V41_FLASH_FP4.cfg, dim=256, moe_inter_dim=128, n_routed_experts=48),
        T=97, x_scale=20.0),
    "softmax_groups_nobias": Workload(
        "softmax_groups_nobias",
        MoEConfig(dim=256, n_routed_experts=64, n_activated_experts=6, moe_inter_dim=192,
                  n_expert_groups=4, n_limited_groups=2, score_func="softmax"),
        T=150),
    "dense_router_ragged": Workload(
        "dense_router_ragged",
        replace(V3_PREFILL.cfg, dim=512, moe_inter_dim=128, n_routed_experts=64),
        T=1100, description="1024+ tokens: GEMM-kernel router (last tile 12 rows), chunked permute"),
    "dense32_router": Workload(
        "dense32_router",
        replace(V3_PREFILL.cfg, dim=1024, moe_inter_dim=128),
        T=1030, description="1024+ tokens, 256 experts: 32x32x16 score GEMM split 4 ways over "
                            "the inputs (last row tile 6 rows)"),
    "split_router_e48": Workload(
        "split_router_e48",
        MoEConfig(dim=256, n_routed_experts=48, n_activated_experts=6, moe_inter_dim=128,
                  score_func="sigmoid", route_scale=1.0, has_bias=True),
        T=1030, description="1024+ tokens with E % 64 != 0: split router, chunked permute"),
    "v3_narrow_2050": Workload(
        "v3_narrow_2050",
        replace(V3_PREFILL.cfg, dim=256, moe_inter_dim=128, n_routed_experts=64),
        T=2050, description="2048+ tokens at narrow widths: many chunks in the permutation, "
                            "ragged last row tile of the score GEMM"),
    "noshared_2051": Workload(
        "noshared_2051",
        MoEConfig(dim=192, n_routed_experts=16, n_activated_experts=3, moe_inter_dim=128,
                  n_shared_experts=0, score_func="sigmoid", route_scale=1.0, has_bias=True),
        T=2051, description="2048+ tokens, no shared expert, width 192 (a combine lane "
                            "group of 256 covers less than one row)"),
    # limits and degenerate cases
    "max_e512_k16": Workload(
        "max_e512_k16",
        MoEConfig(dim=256, n_routed_experts=512, n_activated_experts=16, moe_inter_dim=128,
                  n_expert_groups=16, n_limited_groups=8, score_func="sigmoid", route_scale=2.5,
                  has_bias=True),
        T=100, description="learned routing at the largest E and k: 512 experts, 16 groups, top-16"),
    "single_expert": Workload(
        "single_expert",
        MoEConfig(dim=256, n_routed_experts=1, n_activated_experts=1, moe_inter_dim=128,
                  score_func="softmax"),
        T=50, description="E = k = 1: every token to expert 0 with weight 1 (a dense SwiGLU)"),
    "fp4_one_token": Workload(
        "fp4_one_token",
        replace(V41_FLASH_FP4.cfg, dim=256, moe_inter_dim=128, n_routed_experts=48),
        T=1),
    "ngram_k16": Workload(
        "ngram_k16",
        replace(HASH_BF16.cfg, dim=256, moe_inter_dim=128, n_routed_experts=64, vocab_size=2048,
                n_activated_experts=16, route_mode="ngram"),
        T=130, seq_len=40, description="2-gram hash with 16 primes (duplicates frequent)"),
    "hash_vocab1": Workload(
        "hash_vocab1",
        replace(HASH_BF16.cfg, dim=256, moe_inter_dim=128, n_routed_experts=16, vocab_size=1),
        T=70, description="one-token vocabulary: every token has the same k experts"),
    "sigmoid_noshared_big_tiles": Workload(
        "sigmoid_noshared_big_tiles",
        MoEConfig(dim=320, n_routed_experts=8, n_activated_experts=2, moe_inter_dim=128,
                  n_shared_experts=0, score_func="sigmoid", route_scale=1.5, has_bias=True),
        T=1000),
}
