"""Seeded synthetic workloads for the DFlash drafter pass.

This module only *produces inputs*: shapes, weights, target-layer features, context lengths, page tables,
anchor tokens and the random draws used to build target-token sequences.  It holds none of the drafter's
arithmetic, so both the CPU oracle (through the tests) and the HIP path are fed from it without sharing
any computation.

Shapes follow the workloads the DFlash pages evaluate: Qwen3-4B / Qwen3-8B / LLaMA-3.1-8B targets, a
5-layer drafter, block 16, features from 5 target layers ("DFlash: Block Diffusion for Flash Speculative
Decoding", paper-graph summary, §3.4.3 and §5 implementation details).  Every tensor is synthetic:

* matrices N(0, 0.02) drawn in float32 and rounded to bfloat16 (float32 kept for the tiny fp32 drafter);
* RMSNorm gains 1;
* target hidden-state features N(0, 1);
* target tokens equal a given greedy argmax with probability p, else a uniform token.

Random bits come from Philox4x32-10 (``philox_gen.c``), keyed by (0xDF1A5, config id) and one stream id
per tensor, so every value is reproducible on any machine and independent of thread count.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import subprocess
from typing import Dict, List, Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "_philox_gen.so")
_SRC = os.path.join(_HERE, "philox_gen.c")

BASE_SEED = 0xDF1A5

# stream ids (each tensor / draw has its own Philox stream)
S_WEIGHTS = 1_000
S_FEATURES = 2_000_000
S_CTX_LEN = 3
S_PAGE_PERM = 4
S_BERNOULLI = 5
S_TARGET_TOK = 6
S_ANCHOR = 7
S_ACCEPT_P = 8


def build_generator(force: bool = False) -> str:
    """Compile the Philox generator with gcc (OpenMP) into workloads/_philox_gen.so."""
    if force or not os.path.exists(_SO) or os.path.getmtime(_SO) < os.path.getmtime(_SRC):
        tmp = _SO + ".tmp"
        subprocess.check_call(["gcc", "-O3", "-fopenmp", "-fPIC", "-shared", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _SO)
    return _SO


_lib = None


def _gen():
    global _lib
    if _lib is None:
        if not os.path.exists(_SO):
            build_generator()
        lib = ctypes.CDLL(_SO)
        lib.synth_u32.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                  ctypes.c_void_p]
        lib.synth_normal.argtypes = [ctypes.c_uint64, ctypes.c_uint64, ctypes.c_int64, ctypes.c_int64,
                                     ctypes.c_double, ctypes.c_int, ctypes.c_void_p]
        lib.synth_philox_block.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        _lib = lib
    return _lib


def seed_key(cfg_id: int) -> int:
    return ((BASE_SEED & 0xFFFFFFFF) | ((cfg_id & 0xFFFFFFFF) << 32)) & 0xFFFFFFFFFFFFFFFF


def normal(key: int, stream: int, shape, scale: float, bf16: bool, start: int = 0) -> np.ndarray:
    """N(0, scale^2) samples of stream elements start.. ; bfloat16 results come as uint16 bit patterns."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = np.empty(n, dtype=np.uint16 if bf16 else np.float32)
    if n:
        _gen().synth_normal(key, stream, int(start), n, float(scale), 1 if bf16 else 0, out.ctypes.data)
    return out.reshape(shape)


def philox_block(counter, key) -> np.ndarray:
    """Raw Philox4x32-10 output for a 4-word counter and a 2-word key."""
    c = np.asarray(counter, dtype=np.uint32)
    k = np.asarray(key, dtype=np.uint32)
    out = np.empty(4, dtype=np.uint32)
    _gen().synth_philox_block(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def u32(key: int, stream: int, n: int, start: int = 0) -> np.ndarray:
    out = np.empty(n, dtype=np.uint32)
    if n:
        _gen().synth_u32(key, stream, int(start), n, out.ctypes.data)
    return out


def uniform01(key: int, stream: int, n: int) -> np.ndarray:
    """Uniform [0, 1) doubles from 32-bit words."""
    return u32(key, stream, n).astype(np.float64) / 4294967296.0


def uniform_int(key: int, stream: int, n: int, lo: int, hi: int) -> np.ndarray:
    """Integers in [lo, hi] inclusive (multiply-shift of a 32-bit word)."""
    span = hi - lo + 1
    w = u32(key, stream, n).astype(np.uint64)
    return (lo + ((w * np.uint64(span)) >> np.uint64(32))).astype(np.int64)


def permutation(key: int, stream: int, n: int) -> np.ndarray:
    """A permutation of range(n): sort indices by random 32-bit keys (ties by index)."""
    w = u32(key, stream, n)
    return np.lexsort((np.arange(n), w)).astype(np.int64)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Input formatting helper: bfloat16 bit patterns -> float32 values (exact)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


@dataclasses.dataclass(frozen=True)
class DrafterShape:
    n_layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn: int
    vocab: int
    feat_layers: int
    target_hidden: int
    block_len: int
    rope_theta: float
    rms_eps: float = 1e-6
    bf16: bool = True
    page_size: int = 16

    @property
    def feat_dim(self) -> int:
        return self.feat_layers * self.target_hidden

    @property
    def q_dim(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def kv_dim(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def mask_id(self) -> int:
        return self.vocab - 1


@dataclasses.dataclass(frozen=True)
class Workload:
    """One synthetic workload: a drafter shape plus a batch of requests."""
    cfg_id: int
    name: str
    shape: DrafterShape
    batch: int
    ctx_len: Optional[int]          # fixed context length, or None for per-request random lengths
    ctx_range: Optional[tuple]      # (lo, hi) inclusive, for random lengths
    shuffled_pages: bool
    accept_p: Optional[float]       # fixed acceptance probability, or None for U[p_range]
    accept_p_range: Optional[tuple]
    top_k: int = 8
    ctx_fixed: Optional[tuple] = None   # explicit per-request context lengths (edge cases)
    fc_bias: bool = False               # give the fusion projection a bias fc_b [hidden], N(0, 1)

    # ---------------- seeds ----------------
    @property
    def key(self) -> int:
        return seed_key(self.cfg_id)

    # ---------------- weights ----------------
    def weight_specs(self) -> List[tuple]:
        """(name, shape, kind) in the fixed generation order; kind 'mat' = N(0,0.02), 'gain' = ones."""
        s = self.shape
        specs = [("fc_w", (s.hidden, s.feat_dim), "mat"), ("embed", (s.vocab, s.hidden), "mat")]
        for l in range(s.n_layers):
            specs += [
                (f"l{l}.attn_norm", (s.hidden,), "gain"),
                (f"l{l}.wq", (s.q_dim, s.hidden), "mat"),
                (f"l{l}.wk", (s.kv_dim, s.hidden), "mat"),
                (f"l{l}.wv", (s.kv_dim, s.hidden), "mat"),
                (f"l{l}.wo", (s.hidden, s.q_dim), "mat"),
                (f"l{l}.uk", (s.kv_dim, s.hidden), "mat"),
                (f"l{l}.uv", (s.kv_dim, s.hidden), "mat"),
                (f"l{l}.ffn_norm", (s.hidden,), "gain"),
                (f"l{l}.w_gate", (s.ffn, s.hidden), "mat"),
                (f"l{l}.w_up", (s.ffn, s.hidden), "mat"),
                (f"l{l}.w_down", (s.hidden, s.ffn), "mat"),
            ]
        specs += [("final_norm", (s.hidden,), "gain"), ("lm_head", (s.vocab, s.hidden), "mat")]
        if self.fc_bias:  # last, so that every other tensor keeps its stream
            specs.append(("fc_b", (s.hidden,), "bias"))
        return specs

    def weight(self, idx: int) -> np.ndarray:
        name, shp, kind = self.weight_specs()[idx]
        if kind == "gain":
            if self.shape.bf16:
                return np.full(shp, 0x3F80, dtype=np.uint16)   # 1.0 in bfloat16
            return np.ones(shp, dtype=np.float32)
        # a bias of unit scale moves f by about a third of its own spread (|W_fc x| ~ 0.02 sqrt(feat_dim))
        scale = 1.0 if kind == "bias" else 0.02
        return normal(self.key, S_WEIGHTS + idx, shp, scale, self.shape.bf16)

    def weights(self) -> Dict[str, np.ndarray]:
        """All weights (bfloat16 as uint16 bit patterns, or float32)."""
        return {spec[0]: self.weight(i) for i, spec in enumerate(self.weight_specs())}

    # ---------------- requests ----------------
    def ctx_lens(self) -> np.ndarray:
        if self.ctx_fixed is not None:
            return np.asarray(self.ctx_fixed, dtype=np.int64)
        if self.ctx_len is not None:
            return np.full(self.batch, self.ctx_len, dtype=np.int64)
        lo, hi = self.ctx_range
        return uniform_int(self.key, S_CTX_LEN, self.batch, lo, hi)

    def features(self, r: int, n_rows: int, row0: int = 0) -> np.ndarray:
        """Target-layer hidden states of request r for context tokens row0..row0+n_rows-1, N(0,1).

        Rows are generated from one stream per request, so any row range reproduces the same values.
        """
        s = self.shape
        return normal(self.key, S_FEATURES + r, (n_rows, s.feat_dim), 1.0, s.bf16, start=row0 * s.feat_dim)

    def anchors(self) -> np.ndarray:
        return uniform_int(self.key, S_ANCHOR, self.batch, 0, self.shape.vocab - 2)

    def block_tokens(self) -> np.ndarray:
        """[B, L] int32: anchor then (L-1) mask ids (mask id = vocab-1)."""
        s = self.shape
        bt = np.full((self.batch, s.block_len), s.mask_id, dtype=np.int32)
        bt[:, 0] = self.anchors()
        return bt

    def pages_needed(self, extra_tokens: int = 0) -> np.ndarray:
        ps = self.shape.page_size
        return (self.ctx_lens() + extra_tokens + ps - 1) // ps

    def page_table(self, extra_tokens: int = 0):
        """(page_table [B, max_pages] int32, n_pages): pages of the pool assigned to requests.

        Unused entries are -1.  With shuffled pages the pool is assigned in a random permutation order.
        """
        need = self.pages_needed(extra_tokens)
        n_pages = int(need.sum())
        max_pages = int(max(1, need.max()))
        order = permutation(self.key, S_PAGE_PERM, n_pages) if self.shuffled_pages else np.arange(n_pages)
        pt = np.full((self.batch, max_pages), -1, dtype=np.int32)
        pos = 0
        for r in range(self.batch):
            pt[r, : need[r]] = order[pos: pos + need[r]]
            pos += need[r]
        return pt, max(n_pages, 1)

    def accept_probs(self) -> np.ndarray:
        if self.accept_p is not None:
            return np.full(self.batch, self.accept_p)
        lo, hi = self.accept_p_range
        return lo + (hi - lo) * uniform01(self.key, S_ACCEPT_P, self.batch)

    def target_draws(self):
        """(bernoulli [B, L] bool, random tokens [B, L] int32) used to build target sequences."""
        B, L = self.batch, self.shape.block_len
        u = uniform01(self.key, S_BERNOULLI, B * L).reshape(B, L)
        bern = u < self.accept_probs()[:, None]
        rand = uniform_int(self.key, S_TARGET_TOK, B * L, 0, self.shape.vocab - 1).reshape(B, L).astype(np.int32)
        return bern, rand


def make_target(greedy_tokens: np.ndarray, bern: np.ndarray, rand: np.ndarray) -> np.ndarray:
    """Target tokens Y [B, L]: slot j (j < L-1) compares with the draft at block row j+1; slot L-1 is the
    bonus slot.  Y[:, j] = greedy_tokens[:, j+1] where bern holds, else a uniform token."""
    B, L = greedy_tokens.shape
    y = rand.copy()
    y[:, : L - 1] = np.where(bern[:, : L - 1], greedy_tokens[:, 1:], rand[:, : L - 1])
    return y.astype(np.int32)


TINY = DrafterShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=2, head_dim=64, ffn=768, vocab=4096,
                    feat_layers=3, target_hidden=256, block_len=8, rope_theta=1e6, bf16=False)
QWEN3_4B = DrafterShape(n_layers=5, hidden=2560, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=9728,
                        vocab=151936, feat_layers=5, target_hidden=2560, block_len=16, rope_theta=1e6)
QWEN3_8B = DrafterShape(n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=12288,
                        vocab=151936, feat_layers=5, target_hidden=4096, block_len=16, rope_theta=1e6)
LLAMA31_8B = DrafterShape(n_layers=5, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128, ffn=14336,
                          vocab=128256, feat_layers=5, target_hidden=4096, block_len=16, rope_theta=5e5)

CONFIGS = [
    Workload(0, "tiny-fp32", TINY, 1, 64, None, False, 0.8, None),
    Workload(1, "qwen3-4b-shape", QWEN3_4B, 1, 2048, None, False, 0.85, None),
    Workload(2, "qwen3-8b-shape", QWEN3_8B, 1, 4096, None, False, 0.85, None),
    Workload(3, "qwen3-8b-shape-serve16", QWEN3_8B, 16, None, (512, 8192), True, None, (0.6, 0.95)),
    Workload(4, "llama3.1-8b-shape-32k", LLAMA31_8B, 1, 32768, None, False, 0.8, None),
]

# Reduced shapes for live oracle parity: several GEMM / vocab tiles, ragged vocab and context tails.
SMALL_BF16 = DrafterShape(n_layers=2, hidden=512, n_q_heads=8, n_kv_heads=2, head_dim=128, ffn=1280,
                          vocab=5003, feat_layers=3, target_hidden=512, block_len=16, rope_theta=1e6)
SMALL_GQA8 = DrafterShape(n_layers=1, hidden=256, n_q_heads=8, n_kv_heads=1, head_dim=128, ffn=512,
                          vocab=1000, feat_layers=2, target_hidden=256, block_len=12, rope_theta=1e4)
SMALL_FP32 = DrafterShape(n_layers=2, hidden=128, n_q_heads=4, n_kv_heads=1, head_dim=32, ffn=200,
                          vocab=777, feat_layers=2, target_hidden=96, block_len=5, rope_theta=1e4, bf16=False)
# head_dim 64 in bfloat16: four, eight and one query heads per KV head
SMALL_BF16_D64 = dataclasses.replace(SMALL_BF16, head_dim=64)
SMALL_GQA8_D64 = DrafterShape(n_layers=1, hidden=256, n_q_heads=8, n_kv_heads=1, head_dim=64, ffn=512,
                              vocab=1000, feat_layers=2, target_hidden=256, block_len=12, rope_theta=1e4)
SMALL_MHA_D64 = DrafterShape(n_layers=2, hidden=256, n_q_heads=4, n_kv_heads=4, head_dim=64, ffn=768,
                             vocab=2053, feat_layers=2, target_hidden=256, block_len=16, rope_theta=1e6)

SMALL = [
    Workload(100, "small-bf16-b1", SMALL_BF16, 1, 100, None, False, 0.8, None),
    Workload(101, "small-bf16-paged-b2", SMALL_BF16, 2, None, (1, 300), True, None, (0.6, 0.95)),
    Workload(102, "small-gqa8-b2", SMALL_GQA8, 2, None, (1, 70), True, 0.7, None, top_k=5),
    Workload(103, "small-fp32-b2", SMALL_FP32, 2, None, (0, 40), True, 0.9, None, top_k=3),
    Workload(104, "small-bf16-edge-b2", SMALL_BF16, 2, None, None, True, 0.9, None, top_k=1, ctx_fixed=(0, 33)),
    Workload(105, "small-bf16-long-b1", SMALL_BF16, 1, 1000, None, True, 0.8, None),
    # more than 32 block rows: tiled GEMMs and the tiled LM head (two row tiles, ragged)
    Workload(106, "small-bf16-serve9", SMALL_BF16, 9, None, (0, 400), True, None, (0.6, 0.95)),
    Workload(107, "small-gqa8-b3", SMALL_GQA8, 3, None, (1, 70), True, 0.7, None, top_k=5),
    # the block-size sweep (L in {4, 8, 10}; 16 is the default above)
    Workload(108, "small-bf16-l4-b2", dataclasses.replace(SMALL_BF16, block_len=4), 2, None, (1, 200), True, 0.8,
             None, top_k=4),
    Workload(109, "small-bf16-l8-b2", dataclasses.replace(SMALL_BF16, block_len=8), 2, None, (1, 200), True, 0.8,
             None),
    Workload(110, "small-bf16-l10-b3", dataclasses.replace(SMALL_BF16, block_len=10), 3, None, (1, 200), True,
             None, (0.6, 0.95)),
    # the optional fusion bias ([DF] §3.4.3 "Feature fusion": the projection may carry one)
    Workload(111, "small-bf16-bias-b2", SMALL_BF16, 2, None, (1, 300), True, None, (0.6, 0.95), fc_bias=True),
    Workload(112, "small-fp32-bias-b1", SMALL_FP32, 1, 37, None, True, 0.9, None, top_k=3, fc_bias=True),
    # head_dim 64 (bfloat16): paged ragged contexts; eight query heads per KV head; plain multi-head attention
    Workload(113, "small-bf16-d64-b2", SMALL_BF16_D64, 2, None, (1, 300), True, None, (0.6, 0.95)),
    Workload(114, "small-gqa8-d64-b2", SMALL_GQA8_D64, 2, None, (1, 150), True, 0.7, None, top_k=5),
    Workload(115, "small-mha-d64-b1", SMALL_MHA_D64, 1, 200, None, True, 0.8, None),
]

# Full-size parity cases beyond the five benchmark configurations (expected values in tests/golden/): the
# Qwen3-8B shape with a fusion bias, and 4096 + 1000 context rows, which one inject call runs as a whole
# chunk and a short last chunk.
FULL_EXTRA = [
    Workload(20, "qwen3-8b-shape-bias-5096", QWEN3_8B, 1, 5096, None, True, 0.85, None, fc_bias=True),
]


def by_name(name: str) -> Workload:
    for w in CONFIGS + SMALL + FULL_EXTRA:
        if w.name == name:
            return w
    raise KeyError(name)
