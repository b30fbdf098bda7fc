"""Workload recipes: shapes, distributions and seeds of the synthetic inputs.

The five named workloads c0-c4 follow the layer shapes the pages benchmark (Qwen3-30B-A3B
gate_up 1536x2048, Kimi-K2.5 gate_up 4096x7168 and down 7168x2048, Appendix D.2 Table 8)
with seeded synthetic tokens and weights; c3_mlp is the decode-size layer on the c3 shapes timed
from bf16 tokens to bf16 outputs (Table 11 times such layers); the extra small cases exist for
parity tests.
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    name: str
    E: int                 # experts
    K: int                 # contraction (gate_up: hidden size)
    N: int                 # output rows of the (first) projection
    T: int                 # tokens
    k: int                 # top-k
    routing: str           # "uniform" | "zipf"
    act_dist: str = "normal"   # "normal" | "student_t"
    act_nu: int = 4
    w_std: float = 0.02
    zipf_s: float = 1.1
    zipf_zero: int = 0     # least popular ranks given zero popularity
    seed: int = 0
    # second projection (down) shape, for the decode pair and the full MLP
    N2: int = 0
    K2: int = 0
    mlp: bool = False      # gate_up -> SiLU(gate)*up -> requant -> down -> combine
    x_bf16: bool = False   # tokens handed over in bf16 (else fp32)
    gamma_h: float = 0.0   # one hand-set tensor scale of the intermediate h (MLP only), 448 / (amax_h / 6)
                           # for amax_h = 2.0 (t_mlp) or 64.0 (c4, c3_mlp); the Kimi workloads' per-expert
                           # scales come from calibration (Eq. 5 of each expert's amax of h)
    desc: str = ""

    @property
    def rows(self):
        return self.T * self.k


CONFIGS = {
    "c0": Config("c0", E=4, K=256, N=128, T=64, k=2, routing="uniform", seed=1234,
                 desc="tiny single-projection grouped GEMM"),
    "c1": Config("c1", E=128, K=2048, N=1536, T=16, k=8, routing="uniform", seed=1235,
                 desc="Qwen3-30B-A3B gate_up, decode"),
    "c2": Config("c2", E=128, K=2048, N=1536, T=4096, k=8, routing="zipf", zipf_zero=4, seed=1236,
                 desc="Qwen3-30B-A3B gate_up, prefill, Zipf(1.1)"),
    "c3": Config("c3", E=384, K=7168, N=4096, T=64, k=8, routing="uniform", act_dist="student_t", seed=1237,
                 N2=7168, K2=2048, desc="Kimi-K2.5 gate_up + down, decode"),
    "c4": Config("c4", E=384, K=7168, N=4096, T=8192, k=8, routing="zipf", act_dist="student_t", seed=1238,
                 N2=7168, K2=2048, mlp=True, gamma_h=42.0, desc="Kimi-K2.5 routed-expert MLP, prefill"),
    # the decode-size routed-expert MLP on the c3 shapes, bf16 tokens in and out
    "c3_mlp": Config("c3_mlp", E=384, K=7168, N=4096, T=64, k=8, routing="uniform", act_dist="student_t",
                     seed=1239, N2=7168, K2=2048, mlp=True, gamma_h=42.0, x_bf16=True,
                     desc="Kimi-K2.5 routed-expert MLP, decode"),
    # small cases for parity tests
    "t_mlp": Config("t_mlp", E=4, K=256, N=512, T=64, k=2, routing="uniform", act_dist="student_t", seed=77,
                    N2=256, K2=256, mlp=True, gamma_h=1344.0, desc="tiny MLP (H=256, I=256)"),
    "t_zipf": Config("t_zipf", E=16, K=512, N=384, T=512, k=4, routing="zipf", zipf_zero=3, seed=78,
                     desc="small Zipf prefill with empty experts and ragged tiles"),
}
