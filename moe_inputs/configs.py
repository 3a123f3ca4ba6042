"""Layer shapes of the five synthetic MoE workloads.

The shapes follow the DeepSeek-V3/R1 MoE layer described in Perplexity's
"Lower latency and higher throughput with multi-node DeepSeek deployment"
(section "Expert parallelism": 256 routed experts, each token sent to 8
different experts, one shared expert on every GPU; section "Multi-token
prediction": query length 2 doubles the rows per request; section
"Quantization": FP8 with 128-wide blocks).

Names say what each workload is:

* ``tiny_f32``        64 tokens, hidden 256, 16 experts top-4, fp32, softmax.
* ``decode16``        16 tokens (batch 8 x query length 2), DeepSeek-V3 sizes, bf16.
* ``decode256``       256 tokens (batch 128 x query length 2), same layer.
* ``prefill8192_ep8`` one EP8 rank's share of a prefill: 8192 tokens routed over
                      the rank's 32 local experts, Zipf(1.1) expert popularity.
* ``clustered2048_fp8`` 2048 tokens, 256 experts, fp8 E4M3 expert weights with
                      1x128 fp32 block scales, routing logits boosted inside
                      16 clusters of 16 experts.
* ``decode16_fp8``, ``decode256_fp8``  the decode shapes with fp8 E4M3 expert
                      weights in the pages' 128 x 128 scale tiles.
"""

from dataclasses import dataclass, replace


@dataclass(frozen=True)
class MoEConfig:
    name: str
    T: int            # tokens
    H: int            # hidden size
    E: int            # routed experts visible to this call
    k: int            # experts per token
    I: int            # routed-expert intermediate size
    I_shared: int     # shared-expert intermediate size (0: no shared expert)
    score: str        # "softmax" or "sigmoid"
    act_dtype: str    # "f32" or "bf16": x, gate weight, output
    w_dtype: str      # "f32", "bf16" or "fp8": expert weights
    routing: str      # "random", "zipf" or "clusters": how the gate data is drawn
    seed: int = 0
    quant_block: int = 128   # fp8 block width along K
    w_block_rows: int = 1    # fp8 weight scale block height: 1 (1 x 128 blocks) or 128 (128 x 128 tiles)
    n_group: int = 1         # group-limited routing: E / n_group consecutive experts per group
    topk_group: int = 1      # groups kept eligible per token
    zipf_s: float = 1.1
    n_clusters: int = 16
    cluster_boost: float = 2.0

    @property
    def P(self) -> int:
        """Number of (token, expert) pairs."""
        return self.T * self.k

    def with_(self, **kw) -> "MoEConfig":
        return replace(self, **kw)


_DS = dict(H=7168, E=256, k=8, I=2048, I_shared=2048, score="sigmoid",
           act_dtype="bf16", w_dtype="bf16", routing="random")

CONFIGS = {
    "tiny_f32": MoEConfig("tiny_f32", T=64, H=256, E=16, k=4, I=128, I_shared=128,
                          score="softmax", act_dtype="f32", w_dtype="f32",
                          routing="random"),
    "decode16": MoEConfig("decode16", T=16, **_DS),
    "decode256": MoEConfig("decode256", T=256, **_DS),
    "prefill8192_ep8": MoEConfig("prefill8192_ep8", T=8192,
                                 **{**_DS, "E": 32, "routing": "zipf"}),
    "clustered2048_fp8": MoEConfig("clustered2048_fp8", T=2048,
                                   **{**_DS, "w_dtype": "fp8",
                                      "routing": "clusters"}),
    # the decode shapes with the pages' fp8 scheme: 128 x 128 weight tiles
    "decode16_fp8": MoEConfig("decode16_fp8", T=16, **{**_DS, "w_dtype": "fp8"}, w_block_rows=128),
    "decode256_fp8": MoEConfig("decode256_fp8", T=256, **{**_DS, "w_dtype": "fp8"}, w_block_rows=128),
}


def get_config(name: str) -> MoEConfig:
    try:
        return CONFIGS[name]
    except KeyError:
        raise KeyError(f"unknown workload {name!r}; known: {sorted(CONFIGS)}") from None
