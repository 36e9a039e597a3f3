"""Seeded synthetic inputs for the verify-side path of budget-aware tree
speculative decoding (BASTION, "Methodik" §1-§3 of the method's pages).

This module only draws random numbers and lays them out.  It computes no step
of the path: no softmax, no top-K, no tree, no attention, no acceptance.  Both
the CPU oracle and the HIP library receive exactly these arrays.

Layouts (all C-contiguous):
  logits   [batch][block][vocab]        float32, or bf16 bits as uint16
  q        [batch][nq_max][hq][d]       bf16 bits (uint16) or float32
  k_ctx    [sum_b L_b][hkv][d]          same dtype as q
  v_ctx    [sum_b L_b][hkv][d]
  k_tree   [batch][nq_max][hkv][d]
  v_tree   [batch][nq_max][hkv][d]
  ctx_offsets int64[batch+1]            sequence b owns rows ctx_offsets[b]..[b+1]-1

nq_max = n_max + 1: the root (the last verified token) plus up to n_max drafts.

The synthetic target model (`target_tokens`) stands in for the verifier's
greedy head.  It is an input of the acceptance step, never a compared output:
the target's greedy token at a node of depth d is drawn from the drafter's own
marginal at position d+1 by inverse CDF on a SplitMix64 hash of the node's
path.  Under that law a node is accepted with probability equal to its path
score, which is what the acceptance surrogate assumes (BASTION "Methodik" §2).
"""
from __future__ import annotations

import dataclasses
import math
from dataclasses import dataclass, field

import numpy as np

# Stream ids of the seeded generators.  Each (config, tensor, sequence) gets its
# own PCG64 stream so that any one sequence can be regenerated on its own.
T_LOGITS, T_SPIKE_IDX, T_SPIKE_MAG, T_SPIKE_ON, T_CTX_LEN, T_Q, T_KCTX, T_VCTX, T_KTREE, T_VTREE = range(10)
T_EMBED, T_WQKV, T_WLM, T_ROWS = range(10, 14)


@dataclass(frozen=True)
class Config:
    """One synthetic workload.  Sizes follow the shapes of the method's
    evaluation models (Qwen3-8B, Llama-3.1-8B: "Experimentelle Ergebnisse")."""

    name: str
    index: int                 # seed namespace
    batch: int
    block: int                 # drafter block positions B
    vocab: int                 # V
    logit_dtype: str           # "f32" | "bf16"
    spike_lo: float            # one token per position raised by U[lo, hi]
    spike_hi: float
    spike_p: float             # probability that a position has the spike
    logit_sigma: float
    topk: int                  # K: branching cap per position
    n_max: int                 # budget cap N (draft nodes, root excluded)
    use_stop: bool             # S(N) adaptive stop, else fixed N = n_max
    cost_a: float              # C(N) = a + b N + c max(0, N - knee)
    cost_b: float
    cost_c: float
    cost_knee: int
    l_ar: float = 1.0
    ahat0: float = 1.0         # the root's contribution to A_hat
    hq: int = 32
    hkv: int = 8
    head_dim: int = 128
    attn_dtype: str = "bf16"   # "f32" | "bf16"
    ctx_law: str = "fixed"     # "fixed" | "uniform" | "lognormal"
    ctx_p0: float = 4096       # fixed length | uniform lo | lognormal median
    ctx_p1: float = 0          # -          | uniform hi | lognormal sigma
    ctx_cap: int = 32768
    attn_law: str = "normal"   # "normal" | "mask_sensitive"
    target_seed: int = 0

    @property
    def nq_max(self) -> int:
        return self.n_max + 1

    @property
    def seed(self) -> int:
        return 1234 + self.index

    def replace(self, **kw) -> "Config":
        return dataclasses.replace(self, **kw)


_QWEN_COST = dict(cost_a=1.0, cost_b=0.005, cost_c=0.03, cost_knee=32)

CONFIGS: dict[str, Config] = {
    "tiny": Config(
        name="tiny", index=0, batch=1, block=8, vocab=32000, logit_dtype="f32",
        spike_lo=2.0, spike_hi=10.0, spike_p=1.0, logit_sigma=2.0, topk=4, n_max=16,
        use_stop=True, cost_a=1.0, cost_b=0.02, cost_c=0.0, cost_knee=0,
        hq=8, hkv=8, head_dim=64, attn_dtype="f32", ctx_law="fixed", ctx_p0=128,
        target_seed=99),
    "qwen3_8b": Config(
        name="qwen3_8b", index=1, batch=1, block=16, vocab=151936, logit_dtype="bf16",
        spike_lo=0.0, spike_hi=12.0, spike_p=1.0, logit_sigma=2.0, topk=8, n_max=64,
        use_stop=True, **_QWEN_COST, ctx_law="fixed", ctx_p0=4096, target_seed=100),
    "batched": Config(
        name="batched", index=2, batch=16, block=16, vocab=151936, logit_dtype="bf16",
        spike_lo=0.0, spike_hi=12.0, spike_p=1.0, logit_sigma=2.0, topk=8, n_max=32,
        use_stop=False, **_QWEN_COST, ctx_law="uniform", ctx_p0=512, ctx_p1=4096,
        target_seed=101),
    "llama31_8b": Config(
        name="llama31_8b", index=3, batch=4, block=16, vocab=128256, logit_dtype="bf16",
        spike_lo=0.0, spike_hi=12.0, spike_p=0.5, logit_sigma=2.0, topk=8, n_max=128,
        use_stop=True, **_QWEN_COST, ctx_law="fixed", ctx_p0=8192, target_seed=102),
    "long": Config(
        name="long", index=4, batch=64, block=16, vocab=151936, logit_dtype="bf16",
        spike_lo=0.0, spike_hi=12.0, spike_p=1.0, logit_sigma=2.0, topk=8, n_max=64,
        use_stop=False, **_QWEN_COST, ctx_law="lognormal", ctx_p0=8192, ctx_p1=0.5,
        ctx_cap=32768, target_seed=103),
}

# 64 independent sequences of the Qwen3-8B shape in one step: the streaming
# rate of the same per-sequence work (one cold batch-1 step is latency-bound).
CONFIGS["qwen3_8b_x64"] = CONFIGS["qwen3_8b"].replace(name="qwen3_8b_x64", index=5, batch=64)

# The Qwen3-8B shape with the tree fixed at its budget (N = 64, 65 query
# rows): the tree-attention roofline at a full tree (the S(N) stop picks
# small trees under this logit law).
CONFIGS["qwen3_8b_tree"] = CONFIGS["qwen3_8b"].replace(name="qwen3_8b_tree", index=6,
                                                        use_stop=False)

# Variants used only as parity cases.
CONFIGS["tiny_fixed"] = CONFIGS["tiny"].replace(name="tiny_fixed", use_stop=False)
# Peaked marginals: S-stop trees reach the budget cap and the full block depth.
CONFIGS["qwen3_8b_stress"] = CONFIGS["qwen3_8b"].replace(
    name="qwen3_8b_stress", index=11, spike_lo=14.0, spike_hi=20.0)
CONFIGS["qwen3_8b_masksens"] = CONFIGS["qwen3_8b"].replace(
    name="qwen3_8b_masksens", index=12, use_stop=False, n_max=64, attn_law="mask_sensitive",
    spike_lo=14.0, spike_hi=20.0)
CONFIGS["tiny_masksens"] = CONFIGS["tiny_fixed"].replace(
    name="tiny_masksens", index=10, attn_law="mask_sensitive")
# Few rows cut into one slice per compute unit, as at the Qwen3-8B shape, but
# two sequences of 8 positions with K = 4 (16 slices per row), and four
# sequences of 16 positions with fewer slices per row (4) than K = 8.
CONFIGS["two_seq_k4"] = CONFIGS["tiny_fixed"].replace(name="two_seq_k4", index=13, batch=2)
# Several short ragged contexts at head dim 128 in bf16 (K = 4, GQA 16/4):
# the verify step then runs the context split inside its first kernel, with
# trees of 7 row groups per KV head (more than one per wave).
CONFIGS["fused_ragged"] = CONFIGS["qwen3_8b"].replace(
    name="fused_ragged", index=15, batch=4, block=4, vocab=32000, topk=4, n_max=24,
    use_stop=False, hq=16, hkv=4, ctx_law="uniform", ctx_p0=1, ctx_p1=1500, target_seed=104)
CONFIGS["few_slices"] = CONFIGS["tiny_fixed"].replace(
    name="few_slices", index=14, batch=4, block=16, vocab=65000, logit_dtype="bf16", topk=8,
    spike_lo=0.0, spike_hi=12.0)


def _rng(cfg: Config, tensor: int, seq: int = 0) -> np.random.Generator:
    ss = np.random.SeedSequence(cfg.seed, spawn_key=(tensor, seq))
    return np.random.Generator(np.random.PCG64(ss))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); returns the
    16-bit patterns as uint16.  Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounding = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + rounding) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# ----------------------------------------------------------------------------
# Drafter logits
# ----------------------------------------------------------------------------

def logits_for_seq(cfg: Config, b: int) -> np.ndarray:
    """float32 [block][vocab] logits of sequence b, before any bf16 rounding:
    iid N(0, sigma^2), and at each position one uniformly chosen token raised
    by U[spike_lo, spike_hi] (present with probability spike_p)."""
    x = _rng(cfg, T_LOGITS, b).standard_normal((cfg.block, cfg.vocab), dtype=np.float32)
    x *= np.float32(cfg.logit_sigma)
    idx = _rng(cfg, T_SPIKE_IDX, b).integers(0, cfg.vocab, size=cfg.block)
    mag = _rng(cfg, T_SPIKE_MAG, b).uniform(cfg.spike_lo, cfg.spike_hi, size=cfg.block)
    on = _rng(cfg, T_SPIKE_ON, b).random(cfg.block) < cfg.spike_p
    rows = np.arange(cfg.block)
    x[rows, idx] += np.where(on, mag, 0.0).astype(np.float32)
    return x


def make_logits(cfg: Config, seqs=None) -> np.ndarray:
    """Logits [len(seqs)][block][vocab] in the config's storage type
    (float32, or bf16 bit patterns as uint16)."""
    seqs = range(cfg.batch) if seqs is None else seqs
    out_dt = np.float32 if cfg.logit_dtype == "f32" else np.uint16
    out = np.empty((len(seqs), cfg.block, cfg.vocab), dtype=out_dt)
    for i, b in enumerate(seqs):
        x = logits_for_seq(cfg, b)
        out[i] = x if cfg.logit_dtype == "f32" else f32_to_bf16_bits(x)
    return out


def logits_as_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    return (arr.astype(np.float64) if dtype == "f32" else bf16_bits_to_f32(arr).astype(np.float64))


# ----------------------------------------------------------------------------
# Attention inputs
# ----------------------------------------------------------------------------

def ctx_lengths(cfg: Config) -> np.ndarray:
    r = _rng(cfg, T_CTX_LEN)
    if cfg.ctx_law == "fixed":
        lens = np.full(cfg.batch, int(cfg.ctx_p0), dtype=np.int64)
    elif cfg.ctx_law == "uniform":
        lens = r.integers(int(cfg.ctx_p0), int(cfg.ctx_p1) + 1, size=cfg.batch).astype(np.int64)
    elif cfg.ctx_law == "lognormal":
        ln = r.normal(math.log(cfg.ctx_p0), cfg.ctx_p1, size=cfg.batch)
        lens = np.clip(np.rint(np.exp(ln)), 1, cfg.ctx_cap).astype(np.int64)
    else:
        raise ValueError(cfg.ctx_law)
    return lens


def ctx_offsets(cfg: Config, lens=None) -> np.ndarray:
    lens = ctx_lengths(cfg) if lens is None else lens
    off = np.zeros(len(lens) + 1, dtype=np.int64)
    off[1:] = np.cumsum(lens)
    return off


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    return x.astype(np.float32) if dtype == "f32" else f32_to_bf16_bits(x)


def attn_inputs_for_seq(cfg: Config, b: int, length: int) -> dict:
    """Q, context K/V and tree K/V of sequence b, in storage type.

    "normal": every element iid N(0,1).
    "mask_sensitive": all query rows of a sequence share one direction u, the
    tree keys are c*u with c chosen so that a query-tree score is about 20
    while query-context scores stay O(1), and the context values are tiny.
    Each output row is then close to the mean of the tree values that its
    mask admits, so a single wrong mask bit moves it far beyond tolerance."""
    d, hq, hkv, nq = cfg.head_dim, cfg.hq, cfg.hkv, cfg.nq_max
    q = _rng(cfg, T_Q, b).standard_normal((nq, hq, d), dtype=np.float32)
    kc = _rng(cfg, T_KCTX, b).standard_normal((length, hkv, d), dtype=np.float32)
    vc = _rng(cfg, T_VCTX, b).standard_normal((length, hkv, d), dtype=np.float32)
    kt = _rng(cfg, T_KTREE, b).standard_normal((nq, hkv, d), dtype=np.float32)
    vt = _rng(cfg, T_VTREE, b).standard_normal((nq, hkv, d), dtype=np.float32)
    if cfg.attn_law == "mask_sensitive":
        u = q[0, 0].copy()
        q = (u[None, None, :] + np.float32(0.05) * q).astype(np.float32)
        c = np.float32(20.0 / math.sqrt(d))
        kt = (c * u[None, None, :] + np.float32(0.05) * kt).astype(np.float32)
        vc *= np.float32(1e-3)
    elif cfg.attn_law != "normal":
        raise ValueError(cfg.attn_law)
    s = cfg.attn_dtype
    return dict(q=_store(q, s), k_ctx=_store(kc, s), v_ctx=_store(vc, s),
                k_tree=_store(kt, s), v_tree=_store(vt, s))


def make_attn_inputs(cfg: Config, seqs=None) -> dict:
    """Attention inputs for the given sequences (all by default), concatenated
    in the module-level layouts; ctx_offsets index the concatenated context."""
    lens_all = ctx_lengths(cfg)
    seqs = list(range(cfg.batch)) if seqs is None else list(seqs)
    lens = lens_all[seqs]
    parts = [attn_inputs_for_seq(cfg, b, int(lens_all[b])) for b in seqs]
    out = {k: np.concatenate([p[k] for p in parts], axis=0) if k in ("k_ctx", "v_ctx")
           else np.stack([p[k] for p in parts], axis=0) for k in parts[0]}
    out["ctx_offsets"] = ctx_offsets(cfg, lens)
    out["ctx_len"] = lens
    return out


def attn_scale(cfg: Config) -> float:
    return 1.0 / math.sqrt(cfg.head_dim)


# ----------------------------------------------------------------------------
# Synthetic target model (input of the acceptance step)
# ----------------------------------------------------------------------------

_M64 = (1 << 64) - 1


def splitmix64(x: int) -> int:
    """SplitMix64 output function (Steele, Lea, Flood, OOPSLA 2014): add the
    golden-ratio increment, then the two xor-shift-multiply rounds."""
    z = (x + 0x9E3779B97F4A7C15) & _M64
    z = ((z ^ (z >> 30)) * 0xBF58476D1CE4E5B9) & _M64
    z = ((z ^ (z >> 27)) * 0x94D049BB133111EB) & _M64
    return z ^ (z >> 31)


def path_hash(seed: int, seq: int, path: tuple) -> int:
    h = splitmix64(seed & _M64)
    for w in (seq, len(path)) + tuple(path):
        h = splitmix64(h ^ (int(w) & _M64))
    return h


def path_uniform(seed: int, seq: int, path: tuple) -> float:
    """U in [0,1) from the top 53 bits of the path hash."""
    return (path_hash(seed, seq, path) >> 11) * (1.0 / (1 << 53))


def _splitmix64_np(x: np.ndarray) -> np.ndarray:
    z = x + np.uint64(0x9E3779B97F4A7C15)
    z = (z ^ (z >> np.uint64(30))) * np.uint64(0xBF58476D1CE4E5B9)
    z = (z ^ (z >> np.uint64(27))) * np.uint64(0x94D049BB133111EB)
    return z ^ (z >> np.uint64(31))


def path_uniforms(seeds: np.ndarray, seq: int, path: tuple) -> np.ndarray:
    """path_uniform for many seeds at once (uint64 arithmetic wraps mod 2^64)."""
    with np.errstate(over="ignore"):
        h = _splitmix64_np(np.asarray(seeds, dtype=np.uint64))
        for w in (seq, len(path)) + tuple(path):
            h = _splitmix64_np(h ^ np.uint64(int(w) & _M64))
    return (h >> np.uint64(11)).astype(np.float64) * (1.0 / (1 << 53))


class TargetModel:
    """Greedy token of the synthetic target at any node of a draft tree.

    For a node at depth d (root: d = 0) whose path is (t_1..t_d), the token is
    the smallest v with CDF_{d+1}(v) > U * CDF_{d+1}(V-1), where CDF_{d+1} is
    the float64 running sum, in token-id order, of the unnormalised weights
    exp(l - max l) of the drafter's logits at position d+1 (position B is used
    for d = B), and U = path_uniform(seed, seq, path).
    """

    def __init__(self, cfg: Config, logits_f64: np.ndarray, seqs=None, seed=None):
        self.cfg = cfg
        self.seed = cfg.target_seed if seed is None else seed
        self.seqs = list(range(logits_f64.shape[0])) if seqs is None else list(seqs)
        self._cdf = {}
        self._lf = logits_f64

    def _cdf_for(self, i: int, pos: int) -> np.ndarray:
        key = (i, pos)
        if key not in self._cdf:
            row = self._lf[i, pos]
            w = np.exp(row - row.max())
            self._cdf[key] = np.cumsum(w)
        return self._cdf[key]

    def token(self, i: int, path: tuple, u: float | None = None) -> int:
        pos = min(len(path), self.cfg.block - 1)
        cdf = self._cdf_for(i, pos)
        if u is None:
            u = path_uniform(self.seed, self.seqs[i], path)
        return int(np.searchsorted(cdf, u * cdf[-1], side="right"))

    def tree_targets(self, i: int, node_token, node_parent, n_nodes: int, n_max: int) -> np.ndarray:
        """int32[n_max+1]: target token at every node 0..n_nodes (root = 0), -1 beyond."""
        out = np.full(n_max + 1, -1, dtype=np.int32)
        paths = [()]
        for j in range(1, n_nodes + 1):
            paths.append(paths[int(node_parent[j])] + (int(node_token[j]),))
        for j in range(n_nodes + 1):
            out[j] = self.token(i, paths[j])
        return out


def target_tokens(cfg: Config, logits_f64: np.ndarray, node_token, node_parent, n_nodes,
                  seqs=None, seed=None) -> np.ndarray:
    """int32[batch][n_max+1] target tokens for a batch of trees."""
    tm = TargetModel(cfg, logits_f64, seqs=seqs, seed=seed)
    nb = logits_f64.shape[0]
    out = np.full((nb, node_token.shape[1]), -1, dtype=np.int32)
    for i in range(nb):
        out[i] = tm.tree_targets(i, node_token[i], node_parent[i], int(n_nodes[i]),
                                 node_token.shape[1] - 1)
    return out


# ----------------------------------------------------------------------------
# Weights of the one-layer verification stand-in (random, seeded)
# ----------------------------------------------------------------------------

@dataclass(frozen=True)
class LayerShape:
    """Shape of the verification stand-in: Qwen3-8B's hidden size, heads and
    vocabulary by default (the attention output of all query heads, hq * d,
    is the hidden state the LM head reads)."""
    vocab: int = 151936
    hq: int = 32
    hkv: int = 8
    head_dim: int = 128
    rope_base: float = 1e6

    @property
    def hidden(self) -> int:
        return self.hq * self.head_dim

    @property
    def qkv_out(self) -> int:
        return (self.hq + 2 * self.hkv) * self.head_dim


def layer_shape(cfg: Config) -> LayerShape:
    return LayerShape(vocab=cfg.vocab, hq=cfg.hq, hkv=cfg.hkv, head_dim=cfg.head_dim)


def _normal_lut(scale: float) -> np.ndarray:
    """256 bf16 bit patterns: the N(0, scale^2) quantiles at (i + 0.5) / 256."""
    from statistics import NormalDist
    nd = NormalDist()
    v = np.array([nd.inv_cdf((i + 0.5) / 256) * scale for i in range(256)], np.float32)
    return f32_to_bf16_bits(v)


def _table(cfg: Config, tensor: int, rows: int, cols: int, scale: float) -> np.ndarray:
    """[rows][cols] bf16 bits: each element one of 256 normal quantiles of
    standard deviation `scale`, drawn uniformly (one random byte each)."""
    codes = _rng(cfg, tensor).integers(0, 256, size=(rows, cols), dtype=np.uint8)
    return _normal_lut(scale)[codes]


def layer_weights(cfg: Config, shape: LayerShape | None = None) -> dict:
    """Embedding table embed [vocab][hidden] (std 1), projection w_qkv
    [(hq + 2 hkv) d][hidden] and LM head w_lm [vocab][hidden] (std
    1/sqrt(hidden), so projections and logits are of order 1); bf16 bits."""
    sh = layer_shape(cfg) if shape is None else shape
    H = sh.hidden
    return dict(embed=_table(cfg, T_EMBED, sh.vocab, H, 1.0),
                w_qkv=_table(cfg, T_WQKV, sh.qkv_out, H, 1.0 / math.sqrt(H)),
                w_lm=_table(cfg, T_WLM, sh.vocab, H, 1.0 / math.sqrt(H)))


def hidden_rows(cfg: Config, rows: int, hidden: int) -> np.ndarray:
    """[batch][rows][hidden] bf16 bits, std 1: stand-in final hidden states."""
    return _table(cfg, T_ROWS, cfg.batch * rows, hidden, 1.0).reshape(cfg.batch, rows, hidden)
