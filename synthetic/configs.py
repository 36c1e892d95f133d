"""Workload shapes of the five synthetic decode workloads.

C1  tiny single-layer decode, L=300, 8 query / 2 KV heads, head dim 64, E=512, d'=16
C2  Llama-3.1-8B-shaped single consumer layer, B=1, L=65536, budget 8192
C3  the C2 shapes over 32 layer caches, B=8, prediction interval 16
C4  long context, B=1, L=262144, 32 layers, r=2, heavy-tailed scores
C5  Qwen2.5-7B-shaped, 28 layers, B=4, ragged L in [65536, 131072], interval 8
"""
from dataclasses import dataclass, field


@dataclass(frozen=True)
class Config:
    cid: int
    name: str
    B: int
    L: int            # context length (including the decode token), max over batch
    Hq: int
    Hkv: int
    D: int
    E: int
    Eh: int
    dp: int
    S: int            # sink
    W: int            # local window
    K: int            # important budget
    r: int            # neighbour radius
    layers: int = 1
    interval: int = 1     # prediction interval I
    n_proj: int = 1       # key-projection batch N_p
    producer_stride: int = 4
    n_spans: int = 0
    span_len: int = 0
    alpha: float = 0.0
    ragged: bool = False
    heavy_frac: float = 0.0   # fraction of tokens with shifted affinity
    heavy_shift: float = 0.0
    extra: dict = field(default_factory=dict)

    @property
    def g(self):
        return self.Hq // self.Hkv

    @property
    def n_out(self):
        return self.Hq * self.dp

    @property
    def cap(self):
        return min(self.L, self.S + self.W + self.K)


CONFIGS = {
    1: Config(1, "tiny-L300", B=1, L=300, Hq=8, Hkv=2, D=64, E=512, Eh=128, dp=16,
              S=4, W=16, K=32, r=1, n_spans=3, span_len=4, alpha=3.0),
    2: Config(2, "llama8b-1layer-64k", B=1, L=65536, Hq=32, Hkv=8, D=128, E=4096,
              Eh=1024, dp=32, S=64, W=256, K=7872, r=1, n_spans=64, span_len=8,
              alpha=3.0),
    3: Config(3, "llama8b-32layer-64k-b8", B=8, L=65536, Hq=32, Hkv=8, D=128, E=4096,
              Eh=1024, dp=32, S=64, W=256, K=7872, r=1, layers=32, interval=16,
              n_proj=16),
    4: Config(4, "llama8b-32layer-256k", B=1, L=262144, Hq=32, Hkv=8, D=128, E=4096,
              Eh=1024, dp=32, S=64, W=256, K=7872, r=2, layers=32, interval=16,
              n_proj=16, heavy_frac=0.01, heavy_shift=2.5),
    5: Config(5, "qwen7b-28layer-ragged", B=4, L=131072, Hq=28, Hkv=4, D=128, E=3584,
              Eh=896, dp=32, S=32, W=128, K=3936, r=2, layers=28, interval=8,
              n_proj=8, ragged=True),
}
