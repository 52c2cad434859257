"""Workload shapes and the seeded recipe of every input tensor.

Every tensor has its own stream, keyed by (seed + owner rank, tag). A tensor
owned by rank s (an activation shard, an incoming partial from peer s) uses
seed + s; the local rank's weights use seed + rank. The default seed is 42.

Arrays come back as raw storage bits: uint16 for bf16, uint8 for OCP E4M3FN.
Nothing here computes any part of the method.
"""
from dataclasses import dataclass, field
import math

import numpy as np

from .gen import stream_key, uniform_bf16, normal_bf16, normal_e4m3

SEED = 42


# --------------------------------------------------------------------------
# staged all-gather GEMM: D = alpha * A * B^T + beta * C, A in P row slices
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class AgCase:
    name: str
    M: int
    N: int
    K: int
    P: int
    rank: int = 0
    dtype: str = "bf16"          # operand type of A and B: "bf16" or "e4m3"
    b_layout: str = "nk"         # "nk": B is (N, K) row-major; "kn": (K, N)
    dist: str = "u11"            # "u11": U(-1,1); "n05": clip(0.5 N(0,1), +-448)
    c_dist: str = "u11"          # "u11" or "n01"
    alpha: float = 1.0
    beta: float = 1.0
    swiglu: bool = False         # epilogue silu(u) * v over paired column halves

    @property
    def m(self):
        return self.M // self.P

    @property
    def flop(self):
        return 2.0 * self.M * self.N * self.K


def ag_inputs(case: AgCase, seed: int = SEED):
    """Return dict(a_slices=[P x (m, K)], b=(N,K) or (K,N), c=(M, N out) or None)."""
    m, K, N = case.m, case.K, case.N

    def operand(key, shape):
        if case.dist == "u11":
            assert case.dtype == "bf16"
            return uniform_bf16(key, shape, -1.0, 1.0)
        if case.dist == "n05":
            if case.dtype == "e4m3":
                return normal_e4m3(key, shape, scale=0.5, clip=448.0)
            return normal_bf16(key, shape, 0.0, 0.5)
        if case.dist == "n002":
            assert case.dtype == "bf16"
            return normal_bf16(key, shape, 0.0, 0.02)
        if case.dist == "n01":
            return normal_bf16(key, shape, 0.0, 1.0)
        raise ValueError(case.dist)

    a_slices = [operand(stream_key(seed + s, "ag.a"), (m, K)) for s in range(case.P)]
    bshape = (N, K) if case.b_layout == "nk" else (K, N)
    b = operand(stream_key(seed + case.rank, "ag.b"), bshape)
    n_out = N // 2 if case.swiglu else N
    c = None
    if case.beta != 0.0:
        ckey = stream_key(seed + case.rank, "ag.c")
        if case.c_dist == "u11":
            c = uniform_bf16(ckey, (case.M, n_out), -1.0, 1.0)
        else:
            c = normal_bf16(ckey, (case.M, n_out), 0.0, 1.0)
    return dict(a_slices=a_slices, b=b, c=c)


def ag_rotb_inputs(case: AgCase, seed: int = SEED):
    """Rotating-B all-gather: dict(a=(M, K), b_slices=[P x (n, K) or (K, n)],
    c=(M, N) or None), n = N/P; slice s is rank s's shard of B."""
    n, K = case.N // case.P, case.K

    def operand(key, shape):
        if case.dist == "u11":
            return uniform_bf16(key, shape, -1.0, 1.0)
        if case.dtype == "e4m3":
            return normal_e4m3(key, shape, scale=0.5, clip=448.0)
        return normal_bf16(key, shape, 0.0, 0.5)

    a = operand(stream_key(seed + case.rank, "agb.a"), (case.M, K))
    shape = (n, K) if case.b_layout == "nk" else (K, n)
    b_slices = [operand(stream_key(seed + s, "agb.b"), shape) for s in range(case.P)]
    c = None
    if case.beta != 0.0:
        c = normal_bf16(stream_key(seed + case.rank, "agb.c"), (case.M, case.N), 0.0, 1.0)
    return dict(a=a, b_slices=b_slices, c=c)


# --------------------------------------------------------------------------
# staged GEMM + reduce-scatter dual
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class RsCase:
    name: str
    M: int          # rows of the full partial product (P blocks of M/P)
    N: int
    K: int          # local K shard
    P: int
    rank: int = 0
    b_layout: str = "nk"
    std: float = 0.02
    incoming: bool = True        # seeded N(0,1) partials from the P-1 peers
    alpha: float = 1.0

    @property
    def m(self):
        return self.M // self.P

    @property
    def flop(self):
        return 2.0 * self.M * self.N * self.K


def rs_inputs(case: RsCase, seed: int = SEED):
    """Return dict(a=(M,K), b=(N,K)|(K,N), incoming=[P entries, None at rank])."""
    a = normal_bf16(stream_key(seed + case.rank, "rs.a"), (case.M, case.K), 0.0, case.std)
    bshape = (case.N, case.K) if case.b_layout == "nk" else (case.K, case.N)
    b = normal_bf16(stream_key(seed + case.rank, "rs.b"), bshape, 0.0, case.std)
    incoming = [None] * case.P
    if case.incoming:
        for j in range(case.P):
            if j != case.rank:
                incoming[j] = normal_bf16(stream_key(seed + j, "rs.in"), (case.m, case.N), 0.0, 1.0)
    return dict(a=a, b=b, incoming=incoming)


def rs_tileb_inputs(case: RsCase, seed: int = SEED):
    """Tiled-B reduce-scatter: dict(a, b, incoming) with (M, N/P) partials."""
    a = normal_bf16(stream_key(seed + case.rank, "rsb.a"), (case.M, case.K), 0.0, case.std)
    bshape = (case.N, case.K) if case.b_layout == "nk" else (case.K, case.N)
    b = normal_bf16(stream_key(seed + case.rank, "rsb.b"), bshape, 0.0, case.std)
    incoming = [None] * case.P
    if case.incoming:
        for j in range(case.P):
            if j != case.rank:
                incoming[j] = normal_bf16(stream_key(seed + j, "rsb.in"), (case.M, case.N // case.P), 0.0, 1.0)
    return dict(a=a, b=b, incoming=incoming)


# small parity cases of the column-dual schedules (N/P a multiple of 8)
SMALL_AG_ROTB = [
    AgCase("agb_bf16_p4_small", M=200, N=4 * 64, K=264, P=4, rank=1, dist="u11"),
    AgCase("agb_bf16_p8_kn_small", M=136, N=8 * 40, K=192, P=8, rank=5, b_layout="kn", dist="n05"),
    AgCase("agb_e4m3_p4_small", M=96, N=4 * 56, K=512, P=4, rank=3, dtype="e4m3", dist="n05", beta=0.0),
    AgCase("agb_bf16_p2_medium", M=3000, N=2 * 1024, K=512, P=2, rank=0, dist="u11", alpha=0.5),
    AgCase("agb_bf16_p4_kn_medium", M=2048, N=4 * 512, K=1024, P=4, rank=2, b_layout="kn", dist="n05"),
]
SMALL_RS_TILEB = [
    RsCase("rsb_bf16_p4_small", M=136, N=4 * 64, K=264, P=4, rank=2, std=0.5),
    RsCase("rsb_bf16_p8_kn_small", M=100, N=8 * 48, K=192, P=8, rank=7, b_layout="kn", std=0.5),
    RsCase("rsb_bf16_p4_medium", M=2000, N=4 * 768, K=512, P=4, rank=1, std=0.5),
    # alpha != 1 with incoming partials: alpha scales the own product only
    RsCase("rsb_bf16_p4_alpha_small", M=136, N=4 * 64, K=256, P=4, rank=1, std=0.5, alpha=0.75),
]


# --------------------------------------------------------------------------
# per-token-slot FFN (dispatched input [P*B, L, D], L = T/P slots)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class FfnCase:
    name: str
    B: int
    T: int
    D: int
    k: int
    P: int
    rank: int = 0
    affine: bool = False         # LN gamma ~ U(0.5,1.5), beta ~ U(-0.5,0.5); else 1, 0
    big_bias: bool = False       # biases ~ U(-1,1) instead of the He bound
    eps: float = 1e-5

    @property
    def L(self):
        return self.T // self.P

    @property
    def H(self):
        return self.D * self.k

    @property
    def PB(self):
        return self.P * self.B

    @property
    def flop(self):
        rows = self.PB * self.L
        return 2.0 * rows * self.D * 2 * self.H + 2.0 * rows * self.H * self.D


def he_bound(fan_in):
    """He-uniform bound sqrt(6 / fan_in) (He et al., 2015, uniform variant)."""
    return math.sqrt(6.0 / fan_in)


def ffn_inputs(case: FfnCase, seed: int = SEED):
    s = seed + case.rank
    L, D, H, PB = case.L, case.D, case.H, case.PB
    b1_ = he_bound(D)
    bo_ = he_bound(H)
    x = normal_bf16(stream_key(s, "ffn.x"), (PB, L, D), 0.0, 1.0)
    w1 = uniform_bf16(stream_key(s, "ffn.w1"), (L, D, 2 * H), -b1_, b1_)
    wout = uniform_bf16(stream_key(s, "ffn.wout"), (L, H, D), -bo_, bo_)
    if case.big_bias:
        b1 = uniform_bf16(stream_key(s, "ffn.b1"), (L, 2 * H), -1.0, 1.0)
        bout = uniform_bf16(stream_key(s, "ffn.bout"), (L, D), -1.0, 1.0)
    else:
        b1 = uniform_bf16(stream_key(s, "ffn.b1"), (L, 2 * H), -b1_, b1_)
        bout = uniform_bf16(stream_key(s, "ffn.bout"), (L, D), -bo_, bo_)
    if case.affine:
        gx = uniform_bf16(stream_key(s, "ffn.gx"), (H,), 0.5, 1.5)
        bx = uniform_bf16(stream_key(s, "ffn.bx"), (H,), -0.5, 0.5)
        gg = uniform_bf16(stream_key(s, "ffn.gg"), (H,), 0.5, 1.5)
        bg = uniform_bf16(stream_key(s, "ffn.bg"), (H,), -0.5, 0.5)
    else:
        one = np.full((H,), 0x3F80, dtype=np.uint16)     # bf16 1.0
        zero = np.zeros((H,), dtype=np.uint16)
        gx, bx, gg, bg = one, zero, one.copy(), zero.copy()
    return dict(x=x, w1=w1, b1=b1, wout=wout, bout=bout, gx=gx, bx=bx, gg=gg, bg=bg)


def ffn_upstream_grad(case: FfnCase, seed: int = SEED):
    """The upstream gradient dY [P*B, L, D], N(0, 1) bf16, from its own stream
    (the p04 statement draws the backward check's gradient from a separate
    generator seeded seed + 7)."""
    return normal_bf16(stream_key(seed + 7 + case.rank, "ffn.dy"), (case.PB, case.L, case.D), 0.0, 1.0)


def permute_sources(B, T, D, P, seed: int = SEED, dtype="bf16"):
    """Per-rank layer inputs [B, T, D] for ranks 0..P-1 (rank s uses seed + s)."""
    if dtype == "bf16":
        return [normal_bf16(stream_key(seed + s, "perm.in"), (B, T, D)) for s in range(P)]
    if dtype == "u8":
        from .gen import _raw
        out = []
        for s in range(P):
            n = B * T * D
            out.append((_raw(stream_key(seed + s, "perm.in8"), 0, n) & np.uint64(0xFF))
                       .astype(np.uint8).reshape(B, T, D))
        return out
    raise ValueError(dtype)


# --------------------------------------------------------------------------
# SwiGLU tensor-parallel block: AG GEMM with silu(u)*v epilogue, then RS GEMM
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class SwigluCase:
    name: str
    S: int          # tokens per sequence shard
    D: int          # model dim
    F: int          # local hidden (w1 and w3 column shards are F wide each)
    P: int
    rank: int = 0
    std: float = 0.02

    @property
    def M(self):
        return self.S * self.P

    @property
    def flop(self):
        return 2.0 * self.M * self.D * 2 * self.F + 2.0 * self.M * self.F * self.D


def swiglu_inputs(case: SwigluCase, seed: int = SEED):
    """x shards [P x (S, D)] N(0,1); w13 (D, 2F) = [w1 | w3]; w2 (F, D)."""
    xs = [normal_bf16(stream_key(seed + s, "sw.x"), (case.S, case.D)) for s in range(case.P)]
    w13 = normal_bf16(stream_key(seed + case.rank, "sw.w13"), (case.D, 2 * case.F), 0.0, case.std)
    w2 = normal_bf16(stream_key(seed + case.rank, "sw.w2"), (case.F, case.D), 0.0, case.std)
    return dict(x_shards=xs, w13=w13, w2=w2)


# --------------------------------------------------------------------------
# several column-parallel projections of one gathered input (fused QKV)
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class AgmCase:
    name: str
    M: int          # gathered rows: P slices of m = M/P
    K: int
    P: int
    ns: tuple       # output widths of the projections, e.g. (Nq, Nk, Nv)
    rank: int = 0
    dtype: str = "bf16"
    alpha: float = 1.0

    @property
    def m(self):
        return self.M // self.P

    @property
    def flop(self):
        return 2.0 * self.M * sum(self.ns) * self.K


def ag_multi_inputs(case: AgmCase, seed: int = SEED):
    """dict(a_slices=[P x (m, K)], bs=[(N_i, K)]): the sequence shards N(0, 1)
    (slice s from rank s's stream) and the projection weights N(0, 0.02)
    (this rank's shards), bf16; e4m3 operands from clip(0.5 N(0,1))."""
    def op(key, shape, std):
        if case.dtype == "e4m3":
            return normal_e4m3(key, shape, scale=0.5, clip=448.0)
        return normal_bf16(key, shape, 0.0, std)
    slices = [op(stream_key(seed + s, "agm.x"), (case.m, case.K), 1.0) for s in range(case.P)]
    bs = [op(stream_key(seed + case.rank, f"agm.w{i}"), (n, case.K), 0.02) for i, n in enumerate(case.ns)]
    return dict(a_slices=slices, bs=bs)


SMALL_AGM = [
    AgmCase("agm_bf16_p4_qkv_small", M=4 * 96, K=264, P=4, ns=(136, 40, 40), rank=1),
    AgmCase("agm_e4m3_p8_qkv_small", M=8 * 64, K=512, P=8, ns=(256, 64, 64), rank=6, dtype="e4m3", alpha=0.5),
    AgmCase("agm_bf16_p2_two_medium", M=2 * 1024, K=1024, P=2, ns=(1032, 520), rank=1),
    AgmCase("agm_bf16_p8_qkv_medium", M=8 * 256, K=2048, P=8, ns=(512, 128, 128), rank=3),
]
# the fused QKV projection of an 8B-class model (32 query heads, 8 KV heads,
# head dim 128, D = 4096) at TP = 8: per rank 512 + 128 + 128 columns, 8192 tokens
QKV = AgmCase("ag_qkv_bf16_p8_8192x768x4096", M=8192, K=4096, P=8, ns=(512, 128, 128))


# --------------------------------------------------------------------------
# weight gradient of the all-gather / reduce-scatter linears
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class WgCase:
    name: str
    M: int          # contraction rows (tokens): P slices of m = M/P
    N: int          # output rows (columns of G)
    K: int          # output columns (columns of X)
    P: int
    rank: int = 0
    gathered: str = "x"     # which operand arrives as P row slices: "x" or "g"
    alpha: float = 1.0

    @property
    def m(self):
        return self.M // self.P

    @property
    def flop(self):
        return 2.0 * self.M * self.N * self.K


def wgrad_inputs(case: WgCase, seed: int = SEED):
    """dict(local, slices): with gathered "x", local is G (M, N) (the output
    gradient, this rank's stream) and slices are X's P row slices (m, K),
    slice s from rank s's stream; with gathered "g", local is X (M, K) and
    slices are G's (m, N). All N(0, 1), bf16."""
    if case.gathered == "x":
        local = normal_bf16(stream_key(seed + case.rank, "wg.g"), (case.M, case.N))
        slices = [normal_bf16(stream_key(seed + s, "wg.x"), (case.m, case.K)) for s in range(case.P)]
    else:
        local = normal_bf16(stream_key(seed + case.rank, "wg.x"), (case.M, case.K))
        slices = [normal_bf16(stream_key(seed + s, "wg.g"), (case.m, case.N)) for s in range(case.P)]
    return dict(local=local, slices=slices)


# small parity cases (m a multiple of 64; N and K multiples of 8 with ragged tiles)
SMALL_WGRAD = [
    WgCase("wg_p4_x_small", M=4 * 64, N=200, K=264, P=4, rank=1),
    WgCase("wg_p8_g_small", M=8 * 64, N=136, K=328, P=8, rank=5, gathered="g", alpha=0.5),
    WgCase("wg_p8_x_wrap", M=8 * 128, N=520, K=264, P=8, rank=3),
    WgCase("wg_p2_x_medium", M=2 * 1024, N=1120, K=2088, P=2, rank=1),
    WgCase("wg_p4_g_medium", M=4 * 512, N=1032, K=1536, P=4, rank=2, gathered="g"),
]


# --------------------------------------------------------------------------
# the five workloads at full size, and small parity variants with ragged tails
# --------------------------------------------------------------------------
C1 = AgCase("ag_bf16_p2_256x256x512", M=256, N=256, K=512, P=2, dtype="bf16",
            dist="u11", c_dist="u11", alpha=1.0, beta=1.0)
C2 = AgCase("ag_e4m3_p8_8192x1024x8192", M=8192, N=1024, K=8192, P=8, dtype="e4m3",
            dist="n05", c_dist="n01", alpha=1.0, beta=1.0)
C2_BETA0 = AgCase("ag_e4m3_p8_8192x1024x8192_beta0", M=8192, N=1024, K=8192, P=8,
                  dtype="e4m3", dist="n05", c_dist="n01", alpha=1.0, beta=0.0)
C3 = RsCase("rs_bf16_p8_8192x8192x3584", M=8192, N=8192, K=3584, P=8)
C4 = FfnCase("ffn_slot_b512_t64_d1280_k6_p8", B=512, T=64, D=1280, k=6, P=8)
C5 = SwigluCase("swiglu_p8_s1024_d4096_f1792", S=1024, D=4096, F=1792, P=8)

SMALL_AG = [
    AgCase("ag_bf16_p2_small", M=2 * 200, N=328, K=520, P=2, dist="u11"),
    AgCase("ag_bf16_p4_kn_small", M=4 * 136, N=264, K=200, P=4, b_layout="kn", dist="u11",
           alpha=0.75, beta=-0.5),
    AgCase("ag_e4m3_p4_small", M=4 * 96, N=200, K=544, P=4, dtype="e4m3", dist="n05",
           c_dist="n01", rank=1),
    AgCase("ag_e4m3_p2_beta0_small", M=2 * 130, N=136, K=256, P=2, dtype="e4m3", dist="n05",
           beta=0.0),
    AgCase("ag_bf16_p8_swiglu_small", M=8 * 40, N=2 * 136, K=264, P=8, b_layout="kn",
           dist="n05", beta=0.0, swiglu=True, rank=3),
    # K * element size a multiple of 128 bytes: the direct-to-LDS mainloop
    AgCase("ag_bf16_p2_dma_small", M=2 * 200, N=328, K=384, P=2, dist="u11", rank=1),
    AgCase("ag_e4m3_p4_dma_small", M=4 * 96, N=200, K=640, P=4, dtype="e4m3", dist="n05",
           c_dist="n01", rank=2),
    AgCase("ag_bf16_p4_dma_swiglu_small", M=4 * 72, N=2 * 200, K=256, P=4, dist="n05", beta=0.0,
           swiglu=True),
    # medium: the single-stage launch takes the 256x256 / 256x128 tiles
    AgCase("ag_bf16_p2_dma_medium", M=2 * 2000, N=4040, K=192, P=2, dist="u11", alpha=0.5, beta=2.0),
    AgCase("ag_e4m3_p2_dma_medium", M=2 * 1500, N=2600, K=256, P=2, dtype="e4m3", dist="n05",
           c_dist="n01"),
    # (K, N) weights, K a multiple of 64: transposing LDS reads of DMA'd B tiles
    AgCase("ag_bf16_p4_kn_dma_small", M=4 * 72, N=200, K=192, P=4, b_layout="kn", dist="u11",
           alpha=1.5, beta=0.5, rank=1),
    AgCase("ag_bf16_p4_kn_dma_swiglu_small", M=4 * 72, N=2 * 136, K=256, P=4, b_layout="kn",
           dist="n05", beta=0.0, swiglu=True, rank=2),
    AgCase("ag_bf16_p2_kn_dma_medium", M=2 * 2000, N=4040, K=128, P=2, b_layout="kn", dist="u11"),
    # long K over a narrow output (the shape class of the fp8 rank share)
    AgCase("ag_e4m3_p4_longk_medium", M=4 * 250, N=520, K=4096, P=4, dtype="e4m3", dist="n05",
           c_dist="n01", rank=1),
    AgCase("ag_bf16_p4_longk_medium", M=4 * 512, N=1000, K=2048, P=4, dist="u11", alpha=0.5, rank=3),
    AgCase("ag_bf16_p2_kn_longk_swiglu", M=2 * 300, N=2 * 512, K=2048, P=2, b_layout="kn", dist="n05",
           beta=0.0, swiglu=True, rank=1),
]
SMALL_RS = [
    RsCase("rs_bf16_p4_small", M=4 * 136, N=264, K=328, P=4, rank=2, std=0.5),
    RsCase("rs_bf16_p2_kn_small", M=2 * 100, N=200, K=136, P=2, rank=0, b_layout="kn", std=0.5),
    RsCase("rs_bf16_p4_dma_small", M=4 * 136, N=264, K=448, P=4, rank=3, std=0.5),
    RsCase("rs_bf16_p4_dma_medium", M=4 * 1000, N=4040, K=128, P=4, rank=1, std=0.5),
    RsCase("rs_bf16_p4_kn_dma_small", M=4 * 100, N=264, K=192, P=4, rank=0, b_layout="kn", std=0.5),
    RsCase("rs_bf16_p4_longk_medium", M=4 * 256, N=768, K=2048, P=4, rank=2, std=0.5),
    # alpha != 1 with incoming partials: alpha scales the own product only
    RsCase("rs_bf16_p4_alpha_small", M=4 * 136, N=264, K=256, P=4, rank=1, std=0.5, alpha=0.75),
    RsCase("rs_bf16_p8_kn_alpha_medium", M=8 * 256, N=1032, K=512, P=8, rank=5, b_layout="kn", std=0.5,
           alpha=-1.5),
]
SMALL_FFN = [
    FfnCase("ffn_public_b4_t16_d128_k2_p2", B=4, T=16, D=128, k=2, P=2),
    FfnCase("ffn_small_affine", B=6, T=16, D=136, k=3, P=4, affine=True, big_bias=True, rank=1),
]
SMALL_SWIGLU = [SwigluCase("swiglu_small", S=72, D=264, F=136, P=4, rank=1, std=0.1),
                SwigluCase("swiglu_dma_small", S=40, D=256, F=192, P=4, rank=3, std=0.1)]
