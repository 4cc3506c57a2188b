"""Seeded synthetic inputs for the Orthrus decode step.

This module draws random numbers and lays them out; it performs none of the
method's arithmetic (no attention, no consensus, no append).  Both the fp64
oracle and the HIP path receive the tensors it returns, so neither side
generates its own inputs.

All draws use ``torch.Generator('cpu')``: fp32 N(0,1), rounded to the target
dtype by round-to-nearest-even.  Seeds are ``1000 * config + tensor id (+ 16 *
layer)`` so every tensor of every configuration is reproducible on any host.

The five workloads are the Qwen3-shaped shapes the method is evaluated on
(the summary's §4 names Qwen3 1.7B/4B/8B and a block of K=32; vocabulary
151,936); their contents are synthetic, standing in for trained weights and
the benchmark suites, which are not used.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import torch

F32, BF16 = "f32", "bf16"
_TORCH_DTYPE = {F32: torch.float32, BF16: torch.bfloat16}

# tensor ids used in seeds
T_Q_DIFF, T_Q_AR, T_KC, T_VC, T_KB_DIFF, T_VB_DIFF, T_KB_AR, T_VB_AR = 1, 2, 3, 4, 5, 6, 7, 8
T_LOGITS, T_LENS, T_PAGES, T_MATCHP = 9, 10, 11, 12


@dataclass(frozen=True)
class Config:
    """Shape of one workload (one layer unless ``layers`` > 1)."""
    cid: int
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    D: int
    K: int
    V: int
    layers: int = 1
    L: int = 0                       # fixed prefix length (contiguous)
    L_range: tuple | None = None     # ragged prefix lengths (paged)
    paged: bool = False
    page_size: int = 16
    p_match: float = 0.8
    p_range: tuple | None = None     # per-request match probability range
    num_splits: int = 0              # 0 = library's choice
    extra: dict = field(default_factory=dict)

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv

    @property
    def scale(self) -> float:
        return self.D ** -0.5

    @property
    def torch_dtype(self):
        return _TORCH_DTYPE[self.dtype]

    def with_(self, **kw) -> "Config":
        d = dict(self.__dict__)
        d.update(kw)
        return Config(**d)


CONFIGS = {
    1: Config(1, "tiny-fp32", F32, B=1, Hq=2, Hkv=1, D=64, K=8, V=1000, L=128, p_match=0.8),
    2: Config(2, "qwen3-1.7b-layer", BF16, B=1, Hq=16, Hkv=8, D=128, K=32, V=151936, L=2048,
              p_match=0.8),
    3: Config(3, "qwen3-8b-36layers", BF16, B=1, Hq=32, Hkv=8, D=128, K=32, V=151936, L=8192,
              layers=36, p_match=0.85),
    4: Config(4, "paged-serving-32req", BF16, B=32, Hq=32, Hkv=8, D=128, K=32, V=151936,
              L_range=(512, 8192), paged=True, page_size=16, p_range=(0.5, 0.95)),
    5: Config(5, "long-context-131k", BF16, B=1, Hq=32, Hkv=8, D=128, K=32, V=151936,
              L=131072, p_match=0.8, num_splits=64),
}
LONG_CONTEXT_K_SWEEP = (4, 8, 16, 32, 64)


def gen(seed: int) -> torch.Generator:
    return torch.Generator().manual_seed(int(seed))


def normal(shape, dtype, seed: int) -> torch.Tensor:
    """N(0,1) drawn in fp32, rounded (RNE) to ``dtype``."""
    x = torch.randn(tuple(shape), generator=gen(seed), dtype=torch.float32)
    return x.to(dtype)


def seed_of(cfg: Config, tensor_id: int, layer: int = 0, salt: int = 0) -> int:
    return 1000 * cfg.cid + tensor_id + 16 * layer + 100000 * salt


def prefix_lengths(cfg: Config, salt: int = 0) -> torch.Tensor:
    """int32 [B] prefix lengths: fixed L, or uniform integers in L_range."""
    if cfg.L_range is None:
        return torch.full((cfg.B,), cfg.L, dtype=torch.int32)
    lo, hi = cfg.L_range
    return torch.randint(lo, hi + 1, (cfg.B,), generator=gen(seed_of(cfg, T_LENS, salt=salt)),
                         dtype=torch.int32)


def page_table(cfg: Config, lens: torch.Tensor, salt: int = 0):
    """Random page table with room for the K appended rows of each request.

    Request b owns ceil((lens[b] + K) / page_size) pages, taken from a random
    permutation of all physical pages; unused entries are -1.
    Returns (table int32 [B, max_pages], num_pages).
    """
    ps = cfg.page_size
    need = [(int(l) + cfg.K + ps - 1) // ps for l in lens]
    lmax = cfg.L_range[1] if cfg.L_range else int(lens.max())
    max_pages = (lmax + cfg.K + ps - 1) // ps
    num_pages = sum(need)
    perm = torch.randperm(num_pages, generator=gen(seed_of(cfg, T_PAGES, salt=salt)))
    table = torch.full((cfg.B, max_pages), -1, dtype=torch.int32)
    pos = 0
    for b, nb in enumerate(need):
        table[b, :nb] = perm[pos:pos + nb].to(torch.int32)
        pos += nb
    return table, num_pages


@dataclass
class LayerInputs:
    """One layer's attention inputs for both views (CPU tensors)."""
    q_diff: torch.Tensor      # [B, K, Hq, D]
    q_ar: torch.Tensor
    k_cache: torch.Tensor     # [B, Hkv, cap, D] or [num_pages, Hkv, page, D]
    v_cache: torch.Tensor
    k_blk_diff: torch.Tensor  # [B, K, Hkv, D]  the diffusion module's own block K/V
    v_blk_diff: torch.Tensor
    k_blk_ar: torch.Tensor    # [B, K, Hkv, D]  the AR view's block K/V (appended)
    v_blk_ar: torch.Tensor


@dataclass
class StepInputs:
    cfg: Config
    lens: torch.Tensor                 # int32 [B]
    page_table: torch.Tensor | None    # int32 [B, max_pages]
    num_pages: int
    capacity: int                      # contiguous rows per (b, head)
    layers: list                       # list[LayerInputs]
    diff_logits: torch.Tensor          # [B, K, V]
    ar_logits: torch.Tensor


def layer_inputs(cfg: Config, layer: int, lens, num_pages: int, capacity: int,
                 salt: int = 0) -> LayerInputs:
    dt = cfg.torch_dtype
    B, K, Hq, Hkv, D = cfg.B, cfg.K, cfg.Hq, cfg.Hkv, cfg.D
    if cfg.paged:
        cshape = (num_pages, Hkv, cfg.page_size, D)
    else:
        cshape = (B, Hkv, capacity, D)
    s = lambda tid: seed_of(cfg, tid, layer, salt)  # noqa: E731
    return LayerInputs(
        q_diff=normal((B, K, Hq, D), dt, s(T_Q_DIFF)),
        q_ar=normal((B, K, Hq, D), dt, s(T_Q_AR)),
        k_cache=normal(cshape, dt, s(T_KC)),
        v_cache=normal(cshape, dt, s(T_VC)),
        k_blk_diff=normal((B, K, Hkv, D), dt, s(T_KB_DIFF)),
        v_blk_diff=normal((B, K, Hkv, D), dt, s(T_VB_DIFF)),
        k_blk_ar=normal((B, K, Hkv, D), dt, s(T_KB_AR)),
        v_blk_ar=normal((B, K, Hkv, D), dt, s(T_VB_AR)),
    )


def consensus_logits(B: int, K: int, V: int, p, dtype, seed: int):
    """AR logits N(0,1); diffusion logits a copy in which each position keeps
    the AR argmax with probability p, and otherwise gets +10 (added in fp32,
    rounded to dtype) on one uniformly chosen token other than the AR argmax.

    ``p`` is a float or a length-B sequence (per-request probability).
    Returns (diff_logits, ar_logits), both [B, K, V] in ``dtype``.
    """
    g = gen(seed)
    ar = torch.randn((B, K, V), generator=g, dtype=torch.float32).to(dtype)
    diff = ar.clone()
    if isinstance(p, (list, tuple)):
        pb = torch.tensor(p, dtype=torch.float64)
    else:
        pb = torch.full((B,), float(p), dtype=torch.float64)
    coin = torch.rand((B, K), generator=g, dtype=torch.float64)
    pick = torch.randint(0, max(V - 1, 1), (B, K), generator=g)
    top = ar.float().argmax(dim=-1)           # input construction only
    for b in range(B):
        for i in range(K):
            if coin[b, i] >= pb[b] and V > 1:
                u = int(pick[b, i])
                if u >= int(top[b, i]):
                    u += 1
                diff[b, i, u] = (ar[b, i, u].float() + 10.0).to(dtype)
    return diff, ar


def match_probabilities(cfg: Config, salt: int = 0):
    if cfg.p_range is None:
        return cfg.p_match
    lo, hi = cfg.p_range
    u = torch.rand((cfg.B,), generator=gen(seed_of(cfg, T_MATCHP, salt=salt)),
                   dtype=torch.float64)
    return (lo + (hi - lo) * u).tolist()


def step_inputs(cfg: Config, layers: int | None = None, salt: int = 0,
                with_logits: bool = True) -> StepInputs:
    """All inputs of one decode step of ``cfg`` (CPU tensors)."""
    nl = cfg.layers if layers is None else layers
    lens = prefix_lengths(cfg, salt)
    if cfg.paged:
        table, num_pages = page_table(cfg, lens, salt)
        capacity = 0
    else:
        table, num_pages = None, 0
        capacity = int(lens.max()) + cfg.K
    lay = [layer_inputs(cfg, l, lens, num_pages, capacity, salt) for l in range(nl)]
    if with_logits:
        diff, ar = consensus_logits(cfg.B, cfg.K, cfg.V, match_probabilities(cfg, salt),
                                    cfg.torch_dtype, seed_of(cfg, T_LOGITS, salt=salt))
    else:
        diff = ar = None
    return StepInputs(cfg, lens, table, num_pages, capacity, lay, diff, ar)


T_LM_HIDDEN, T_LM_WEIGHT = 13, 14


def lmhead_inputs(R: int, H: int, V: int, seed: int = 0):
    """Hidden states [R, H] and an LM-head weight [V, H], bf16.

    The hidden rows are N(0,1); the weight rows N(0,1)/sqrt(H), so that the
    logits are N(0,1)-scaled like a trained head's, with no structure."""
    hidden = normal((R, H), torch.bfloat16, 1000 * 90 + T_LM_HIDDEN + 100000 * seed)
    w = torch.randn((V, H), generator=gen(1000 * 90 + T_LM_WEIGHT + 100000 * seed),
                    dtype=torch.float32)
    return hidden, (w * H ** -0.5).to(torch.bfloat16)


def custom_step(B: int, Hq: int, Hkv: int, D: int, K: int, lens, dtype=BF16, paged=False,
                seed: int = 0, V: int = 1000, p=0.8, extra_capacity: int = 0) -> StepInputs:
    """A small step with explicit per-request prefix lengths (edge cases).

    Contiguous caches get capacity max(lens) + K + extra_capacity; paged ones
    a random page table with room for the K appended rows.
    """
    lens_t = torch.tensor(list(lens), dtype=torch.int32)
    assert lens_t.numel() == B
    cfg = Config(90 + (seed % 10), f"custom-{seed}", dtype, B=B, Hq=Hq, Hkv=Hkv, D=D, K=K, V=V,
                 L_range=(int(lens_t.min()), int(lens_t.max())), paged=paged, p_match=p)
    salt = 1 + seed
    if paged:
        table, num_pages = page_table(cfg, lens_t, salt)
        capacity = 0
    else:
        table, num_pages = None, 0
        capacity = int(lens_t.max()) + K + extra_capacity
    lay = [layer_inputs(cfg, 0, lens_t, num_pages, capacity, salt)]
    diff, ar = consensus_logits(B, K, V, p, cfg.torch_dtype, seed_of(cfg, T_LOGITS, salt=salt))
    return StepInputs(cfg, lens_t, table, num_pages, capacity, lay, diff, ar)


T_MD_Q, T_MD_KC, T_MD_VC, T_MD_KB, T_MD_VB, T_MD_ANCH = 15, 16, 17, 18, 19, 20

# The training-time block mask (M_diff) at the Qwen3-8B attention shape: a
# micro-batch of 4 sequences of 4,096 tokens, K = 32 blocks tiling each
# sequence (the summary's §2.2 selects blocks of length K inside a sequence;
# tiling is the case where every position is trained once).
MDIFF_WORKLOAD = dict(name="mdiff-qwen3-8b-4x4096", B=4, N=4096, K=32, Hq=32, Hkv=8, D=128,
                      layout="tile")


@dataclass
class MdiffInputs:
    """Inputs of one M_diff forward (CPU tensors)."""
    q: torch.Tensor        # [B, NB, K, Hq, D]  the diffusion view's block queries
    k_blk: torch.Tensor    # [B, NB, K, Hkv, D] its block keys
    v_blk: torch.Tensor
    k_ctx: torch.Tensor    # [B, Hkv, N, D]     the clean context (AR view)
    v_ctx: torch.Tensor
    anchors: torch.Tensor  # int32 [B, NB]


def mdiff_anchors(B: int, N: int, K: int, NB: int, layout: str, seed: int) -> torch.Tensor:
    """Anchor positions: "tile" puts block j at j*K (NB = N // K blocks that
    cover the sequence); "random" draws NB positions uniformly in [0, N],
    sorted per sequence (blocks may overlap; 0 and N are allowed)."""
    if layout == "tile":
        a = torch.arange(NB, dtype=torch.int32) * K
        return a.expand(B, NB).contiguous()
    a = torch.randint(0, N + 1, (B, NB), generator=gen(seed), dtype=torch.int64)
    return a.sort(dim=1).values.to(torch.int32)


def mdiff_inputs(B: int, N: int, K: int, Hq: int, Hkv: int, D: int, layout: str = "tile",
                 NB: int = 0, dtype=BF16, seed: int = 0) -> MdiffInputs:
    dt = _TORCH_DTYPE[dtype]
    NB = NB or N // K
    s = lambda tid: 1000 * 95 + tid + 100000 * seed  # noqa: E731
    return MdiffInputs(
        q=normal((B, NB, K, Hq, D), dt, s(T_MD_Q)),
        k_blk=normal((B, NB, K, Hkv, D), dt, s(T_MD_KB)),
        v_blk=normal((B, NB, K, Hkv, D), dt, s(T_MD_VB)),
        k_ctx=normal((B, Hkv, N, D), dt, s(T_MD_KC)),
        v_ctx=normal((B, Hkv, N, D), dt, s(T_MD_VC)),
        anchors=mdiff_anchors(B, N, K, NB, layout, s(T_MD_ANCH)))


T_FP8_KS, T_FP8_VS = 21, 22


def fp8_cache(values: torch.Tensor, seed: int):
    """An OCP E4M3 cache holding about `values`: each row (the last axis) gets
    a random power-of-two scale 2^e, e uniform in {-7, -6, -5}, and codes =
    the E4M3 nearest to value / 2^e (clamped to +-448).  The scales are drawn,
    not derived from the rows, so this is input construction, not the
    quantizer the append uses.  Returns (codes uint8 [..., D], scales float32
    [...])."""
    e = torch.randint(-7, -4, values.shape[:-1], generator=gen(seed)).to(torch.float32)
    sc = torch.exp2(e)
    x = (values.float() / sc[..., None]).clamp(-448.0, 448.0)
    codes = x.to(torch.float8_e4m3fn).view(torch.uint8)
    return codes.contiguous(), sc.contiguous()


T_MODEL = 30


def model_weights(dims, seed: int = 0, device="cpu"):
    """Random weights of a Qwen3-style model (the layer of the decode step,
    see oracle.model) at the given dimensions, bf16, seeded.  Scales keep
    activations O(1): projections N(0, 1/fan_in), norm weights 1 + N(0,
    0.1^2), embeddings N(0, 1).  The diffusion view's attention weights start
    from the AR ones (the agents-report core design: the module is
    initialised from its AR counterparts) plus an independent N(0, 0.2^2 /
    fan_in) change, standing in for its training.  The embedding table has
    one extra row, index V: the <mask> token.  device="cuda" draws on the GPU
    (seeded, for the benchmark's 36-layer model only)."""
    g = torch.Generator(device=device).manual_seed(1000 * 96 + T_MODEL + 100000 * seed)

    def rn(shape, std, mean=0.0):
        x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
        return (x * std + mean).to(torch.bfloat16)

    H, Hq, Hkv, D, I, V = dims.H, dims.Hq, dims.Hkv, dims.D, dims.I, dims.V
    nqkv = (Hq + 2 * Hkv) * D
    w = {"embed": rn((V + 1, H), 1.0), "final_norm": rn((H,), 0.1, 1.0),
         "lm_head": rn((V, H), H ** -0.5)}
    for l in range(dims.layers):
        w[f"l{l}.in_norm"] = rn((H,), 0.1, 1.0)
        w[f"l{l}.post_norm"] = rn((H,), 0.1, 1.0)
        w[f"l{l}.q_norm"] = rn((D,), 0.1, 1.0)
        w[f"l{l}.k_norm"] = rn((D,), 0.1, 1.0)
        w[f"l{l}.ar.wqkv"] = rn((nqkv, H), H ** -0.5)
        w[f"l{l}.ar.wo"] = rn((H, Hq * D), (Hq * D) ** -0.5)
        w[f"l{l}.diff.wqkv"] = (w[f"l{l}.ar.wqkv"].float()
                                + rn((nqkv, H), 0.2 * H ** -0.5).float()).to(torch.bfloat16)
        w[f"l{l}.diff.wo"] = (w[f"l{l}.ar.wo"].float()
                              + rn((H, Hq * D), 0.2 * (Hq * D) ** -0.5).float()).to(torch.bfloat16)
        w[f"l{l}.wgu"] = rn((2 * I, H), H ** -0.5)
        w[f"l{l}.wdown"] = rn((H, I), I ** -0.5)
    return w
