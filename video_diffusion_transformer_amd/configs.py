"""The workloads of one Wan2.2-A14B DiT self-attention step.

Token grids follow the output-spec arithmetic on the AWS Neuron page
"Optimizing High-Quality Offline Video Generation", section "Grounding in an
output spec": 832x480 at 81 frames gives 21 x 30 x 52 = 32,760 tokens, and
1280x720 at 81 frames gives 21 x 45 x 80 = 75,600 tokens (the sequence length
quoted in the TensorRT-LLM pull request "Optimize Wan2.2 Dataflow", Test
Configuration). B = 2 is the classifier-free-guidance pair (conditioned and
unconditioned pass of the same latent). 40 heads x 128 channels is the A14B
attention shape (same AWS page, section "Tensor parallelism").
"""

from dataclasses import dataclass


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    T: int
    H: int
    W: int
    heads: int = 40
    head_dim: int = 128
    seed: int = 0
    dtype: str = "bf16"

    @property
    def S(self):
        return self.T * self.H * self.W

    @property
    def D(self):
        return self.heads * self.head_dim

    def attn_flop(self):
        """Dense bidirectional attention: QK^T and PV, 2 FLOP per MAC."""
        return 4.0 * self.B * self.heads * self.S * self.S * self.head_dim

    def norm_bytes(self):
        """Algorithmic HBM bytes of the in-place norm + RoPE: Q and K read once
        and written once, bf16 (V is not touched)."""
        return 4.0 * self.B * self.S * self.D * 2


WORKLOADS = {
    "tiny": Workload("tiny", B=1, T=2, H=8, W=8, heads=2, seed=0),
    "480p": Workload("480p", B=2, T=21, H=30, W=52, seed=1),
    "720p": Workload("720p", B=2, T=21, H=45, W=80, seed=2),
    "720p_fp8": Workload("720p_fp8", B=2, T=21, H=45, W=80, seed=2, dtype="fp8"),
    "long": Workload("long", B=1, T=31, H=45, W=80, seed=4),
}
