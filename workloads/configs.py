"""The five decode-attention workloads, as plain shapes and seeds.

Each workload is stated by what it is and its sizes.  Seeds: workload k uses
seed k for its tensors; point j of a sweep uses 100*k + j.
"""

from dataclasses import dataclass

__all__ = ["DecodeWorkload", "BifurcatedWorkload", "TINY", "CODELLAMA34B_SHARE",
           "MHA_SWEEP", "BIFURCATED_MQA", "BIFURCATED_GQA", "CODELLAMA34B_SHARE_PAGED",
           "MHA_B16_L65536_PAGED", "CODELLAMA34B_SHARE_FP8", "MHA_B16_L65536_FP8", "ALL_DECODE",
           "ALL_BIFURCATED", "ALL_PAGED", "ALL_FP8", "PrefillWorkload", "PREFILL_CODELLAMA34B_SHARE",
           "PREFILL_MHA", "ALL_PREFILL"]


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    max_len: int
    dtype: str                 # 'bf16' or 'fp32' (q, K, V storage), or 'fp8' (E4M3 K/V codes, bf16 q)
    ragged: bool               # lens uniform in [max_len/2, max_len] when True
    n_splits: int              # <= 0: split count chosen by the planner
    seed: int
    tol: float                 # max-abs error bound against the fp64 oracle
    page_size: int = 0         # > 0: paged cache of pages this many rows long

    def kv_bytes_allocated(self):
        sz = {"bf16": 2, "fp32": 4, "fp8": 1}[self.dtype]
        return 2 * self.batch * self.kv_heads * self.max_len * self.head_dim * sz


@dataclass(frozen=True)
class BifurcatedWorkload:
    name: str
    samples: int
    q_heads: int
    kv_heads: int
    head_dim: int
    ctx_len: int
    dec_max: int
    dec_lo: int                # dec_lens uniform in [dec_lo, dec_max]
    dtype: str
    seed: int
    tol: float


# Tiny check case: batch 1, 4 query heads = 4 KV heads, D 64, 512 tokens,
# fp32, 4 KV splits.
TINY = DecodeWorkload("tiny_b1_h4_d64_l512_fp32", 1, 4, 4, 64, 512, "fp32",
                      False, 4, 1, 1e-5)

# One GPU's quarter-of-heads share of a CodeLlama-34B layer: 16 query heads
# over 2 KV heads (GQA 8:1), D 128, 65536 cached tokens, batch 1, bf16.
CODELLAMA34B_SHARE = DecodeWorkload("codellama34b_share_b1_hq16_hkv2_d128_l65536_bf16",
                                    1, 16, 2, 128, 65536, "bf16", False, 0, 2, 1e-2)

# MHA length sweep: 32 heads = 32 KV heads, D 128, bf16, ragged lengths
# uniform in [L/2, L], L in {512, 2K, 8K, 32K, 64K}, batch 1 and 16.
MHA_SWEEP = tuple(
    DecodeWorkload(f"mha_b{B}_h32_d128_l{L}_bf16", B, 32, 32, 128, L, "bf16", True, 0,
                   100 * 3 + j, 1e-2)
    for j, (L, B) in enumerate((L, B) for L in (512, 2048, 8192, 32768, 65536) for B in (1, 16))
)

# Bifurcated MQA: 64 samples share an 8192-token context, each with 256 decode
# tokens; 32 query heads over 1 KV head, D 128, bf16.
BIFURCATED_MQA = BifurcatedWorkload("bifurcated_mqa_s64_ctx8192_dec256_hq32_hkv1_d128_bf16",
                                    64, 32, 1, 128, 8192, 256, 256, "bf16", 4, 1e-2)

# Bifurcated GQA: 128 samples share a 32768-token context; decode lengths
# uniform in [1, 512]; 32 query heads over 8 KV heads, D 128, bf16.
BIFURCATED_GQA = BifurcatedWorkload("bifurcated_gqa_s128_ctx32768_dec1to512_hq32_hkv8_d128_bf16",
                                    128, 32, 8, 128, 32768, 512, 1, "bf16", 5, 1e-2)

# Paged-cache forms of the 64K workloads: the same shapes with the cache in
# 16-row pages (a common serving block size) handed out in shuffled order.
CODELLAMA34B_SHARE_PAGED = DecodeWorkload("codellama34b_share_paged16_b1_hq16_hkv2_d128_l65536_bf16",
                                          1, 16, 2, 128, 65536, "bf16", False, 0, 6, 1e-2, page_size=16)
MHA_B16_L65536_PAGED = DecodeWorkload("mha_paged16_b16_h32_d128_l65536_bf16", 16, 32, 32, 128, 65536,
                                      "bf16", True, 0, 7, 1e-2, page_size=16)

# E4M3 (fp8) cache forms of the 64K workloads: K and V stored as one-byte
# codes with per-KV-head scales, the query bf16.
CODELLAMA34B_SHARE_FP8 = DecodeWorkload("codellama34b_share_fp8kv_b1_hq16_hkv2_d128_l65536",
                                        1, 16, 2, 128, 65536, "fp8", False, 0, 8, 1e-2)
MHA_B16_L65536_FP8 = DecodeWorkload("mha_fp8kv_b16_h32_d128_l65536", 16, 32, 32, 128, 65536, "fp8", True, 0,
                                    9, 1e-2)

@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    max_len: int
    dtype: str
    seed: int
    tol: float


# Causal prefill of a whole prompt: the CodeLlama-34B one-GPU share over 16K
# tokens, and 32-head MHA over 8K tokens at batch 2.
PREFILL_CODELLAMA34B_SHARE = PrefillWorkload("prefill_codellama34b_share_b1_hq16_hkv2_d128_l16384_bf16", 1, 16, 2,
                                             128, 16384, "bf16", 10, 1e-2)
PREFILL_MHA = PrefillWorkload("prefill_mha_b2_h32_d128_l8192_bf16", 2, 32, 32, 128, 8192, "bf16", 11, 1e-2)
ALL_PREFILL = (PREFILL_CODELLAMA34B_SHARE, PREFILL_MHA)

ALL_DECODE = (TINY, CODELLAMA34B_SHARE) + MHA_SWEEP
ALL_PAGED = (CODELLAMA34B_SHARE_PAGED, MHA_B16_L65536_PAGED)
ALL_FP8 = (CODELLAMA34B_SHARE_FP8, MHA_B16_L65536_FP8)
ALL_BIFURCATED = (BIFURCATED_MQA, BIFURCATED_GQA)
