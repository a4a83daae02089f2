"""Seeded synthetic workloads for the encoder and verification attention path.

This module generates inputs only. It holds none of the attention arithmetic
(no projection, score, softmax or merge), so both the fp64 oracle and the HIP
path can be fed from it without sharing any of the method's code.

Workloads (shapes follow the pages; values are synthetic because the pages'
audio, transcripts and trained weights are not available):

* "audio.cpp PR #1223, Add Edda ASR" (PR description and the encoder commit
  message): a Whisper-large-v3 encoder, one 30 s window = 1500 frames; the
  verification block is an anchor plus up to 15 drafted tokens; beam search
  uses 5 beams sharing one token-tree KV cache whose mask rows admit only a
  beam's ancestors.
* "higgs-audio-v3-stt-GGUF" model card, architecture note: 4 s chunks encoded
  independently with within-chunk attention (4 s = 200 encoder positions at
  50 positions per second).
* "BuzzASR/danish discussion #1": the encoder is fully bidirectional and has
  32 layers ("layer 8 ... layers 9-32"); 1000 mel frames = 500 positions.

Random-number convention: every tensor is drawn from
``numpy.random.default_rng([seed, cfg, layer, tensor_id, trial])`` (PCG64) as
float64 ``standard_normal`` times sigma, then rounded to float16 (round to
nearest even). ``N(0, s)`` in the workload descriptions is read as variance s.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

# Whisper-large-v3 encoder attention geometry.
D_MODEL = 1280
N_HEADS = 20
HEAD_DIM = 64
QKV_COLS = 3 * D_MODEL

# Tensor ids of the RNG key.
T_X, T_WQKV, T_BQ, T_BV, T_WO, T_VALID, T_Q, T_KSELF, T_VSELF, T_KCROSS, T_VCROSS, T_L, T_TREE = range(13)

W_VAR = 1.0 / D_MODEL   # W_qkv and W_o entries: N(0, 1/1280)
B_VAR = 0.02            # q and v biases: N(0, 0.02); no k bias

FRAMES_PER_WINDOW = 1500   # one 30 s window
POSITIONS_PER_SECOND = 50  # 3000 mel frames -> 1500 positions over 30 s
CHUNK_SECONDS = 4
CHUNK_LEN = CHUNK_SECONDS * POSITIONS_PER_SECOND  # 200
ENCODER_LAYERS = 32
VERIFY_BLOCK = 16  # anchor + 15 drafted tokens
BEAMS = 5


def rng_for(seed: int, cfg: int, layer: int, tensor_id: int, trial: int = 0) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(cfg), int(layer), int(tensor_id), int(trial)])


def normal_f16(rng: np.random.Generator, shape, var: float) -> np.ndarray:
    """float64 N(0, var) draw rounded to float16 (numpy's cast is round-to-nearest-even)."""
    return (rng.standard_normal(shape) * math.sqrt(var)).astype(np.float16)


@dataclass
class EncoderLayerWeights:
    w_qkv: np.ndarray          # fp16 [1280, 3840]; column blocks Q | K | V, head h at 64h..64h+63
    b_qkv: np.ndarray          # fp16 [3840]; the K third is zero
    w_o: np.ndarray            # fp16 [1280, 1280]
    b_o: np.ndarray | None = None


def encoder_layer_weights(cfg: int, layer: int, seed: int = 0) -> EncoderLayerWeights:
    w_qkv = normal_f16(rng_for(seed, cfg, layer, T_WQKV), (D_MODEL, QKV_COLS), W_VAR)
    b_qkv = np.zeros(QKV_COLS, dtype=np.float16)
    b_qkv[:D_MODEL] = normal_f16(rng_for(seed, cfg, layer, T_BQ), (D_MODEL,), B_VAR)
    b_qkv[2 * D_MODEL:] = normal_f16(rng_for(seed, cfg, layer, T_BV), (D_MODEL,), B_VAR)
    w_o = normal_f16(rng_for(seed, cfg, layer, T_WO), (D_MODEL, D_MODEL), W_VAR)
    return EncoderLayerWeights(w_qkv=w_qkv, b_qkv=b_qkv, w_o=w_o)


@dataclass
class EncoderWorkload:
    cfg: int
    name: str
    batch: int
    seq_len: int
    chunk_len: int          # 0 = full bidirectional window
    valid_len: np.ndarray   # int32 [batch]; keys at positions >= valid_len are masked
    layers: int
    seed: int = 0
    x: np.ndarray | None = field(default=None, repr=False)  # fp16 [batch*seq_len, 1280]

    @property
    def rows(self) -> int:
        return self.batch * self.seq_len

    def weights(self, layer: int) -> EncoderLayerWeights:
        return encoder_layer_weights(self.cfg, layer, self.seed)


ENCODER_CONFIGS = {
    0: dict(name="one 4 s chunk, 1 sublayer", batch=1, seq_len=CHUNK_LEN, chunk_len=0, layers=1),
    1: dict(name="one 30 s window, 32 sublayers", batch=1, seq_len=FRAMES_PER_WINDOW, chunk_len=0,
            layers=ENCODER_LAYERS),
    2: dict(name="45 s of audio in 4 s chunks, 32 sublayers", batch=1, seq_len=12 * CHUNK_LEN,
            chunk_len=CHUNK_LEN, layers=ENCODER_LAYERS),
    3: dict(name="16 batched 30 s windows with padded key tails, 32 sublayers", batch=16,
            seq_len=FRAMES_PER_WINDOW, chunk_len=0, layers=ENCODER_LAYERS),
}


def encoder_workload(cfg: int, seed: int = 0, layers: int | None = None, batch: int | None = None,
                     seq_len: int | None = None, chunk_len: int | None = None,
                     valid_len=None) -> EncoderWorkload:
    """Build encoder workload `cfg` (0..3). Keyword overrides shrink a workload for tests
    while keeping its structure (same RNG streams, same distributions)."""
    c = dict(ENCODER_CONFIGS[cfg])
    if layers is not None:
        c["layers"] = layers
    if batch is not None:
        c["batch"] = batch
    if seq_len is not None:
        c["seq_len"] = seq_len
    if chunk_len is not None:
        c["chunk_len"] = chunk_len
    b, s = c["batch"], c["seq_len"]
    if valid_len is not None:
        v = np.asarray(valid_len, dtype=np.int32).reshape(b)
    elif cfg == 2:
        # 45 s = 2250 positions: 11 full chunks and 50 valid positions of the 12th.
        v = np.full(b, min(s, 45 * POSITIONS_PER_SECOND), dtype=np.int32)
    elif cfg == 3:
        lo = min(300, s)
        v = rng_for(seed, cfg, 0, T_VALID).integers(lo, s + 1, size=b).astype(np.int32)
    else:
        v = np.full(b, s, dtype=np.int32)
    x = normal_f16(rng_for(seed, cfg, 0, T_X), (b * s, D_MODEL), 1.0)
    return EncoderWorkload(cfg=cfg, name=c["name"], batch=b, seq_len=s, chunk_len=c["chunk_len"],
                           valid_len=v, layers=c["layers"], seed=seed, x=x)


# --------------------------------------------------------------------------------------
# Speculative block verification (decoder self-attention over a KV cache indexed by
# position, plus cross-attention over the 1500 encoder frames).
# --------------------------------------------------------------------------------------

@dataclass
class VerifyCase:
    q: np.ndarray            # fp16 [n_q, 20, 64]
    k: np.ndarray            # fp16 [n_kv, 20, 64]; row = cache slot = position
    v: np.ndarray            # fp16 [n_kv, 20, 64]
    mask: np.ndarray | None  # bool [n_q, n_kv]; True = key admitted; None = every key admitted
    kind: str                # "causal" | "cross" | "tree"
    parents: np.ndarray | None = None  # int32 [n_kv] for "tree": parent slot, -1 at the root
    query_slots: np.ndarray | None = None  # int32 [n_q] for "tree"

    @property
    def n_q(self) -> int:
        return self.q.shape[0]

    @property
    def n_kv(self) -> int:
        return self.k.shape[0]


def verify_cache_lengths(trials: int = 8, seed: int = 0) -> np.ndarray:
    """Self-attention cache length L per trial, uniform on [32, 448]."""
    return np.array([cache_length(t, seed) for t in range(trials)], dtype=np.int32)


def cache_length(trial: int, seed: int = 0) -> int:
    return int(rng_for(seed, 4, 0, T_L, trial).integers(32, 449))


def causal_block_mask(n_q: int, n_kv: int) -> np.ndarray:
    """Mask rows of a block of n_q new tokens that occupy the last n_q cache slots:
    query t sits at position n_kv - n_q + t and admits every slot up to and including it."""
    t = np.arange(n_q)[:, None]
    j = np.arange(n_kv)[None, :]
    return j <= (n_kv - n_q + t)


def beam_tree(n_kv: int, rng: np.random.Generator, beams: int = BEAMS):
    """Token tree of n_kv slots shared by `beams` beams (never copied or reordered).

    A shared prefix chain of P = n_kv - beams*S slots (S = (n_kv - 4) // beams steps)
    is followed by S steps; at every step each beam's newest token takes a fresh slot
    whose parent is the previous step's slot of a beam drawn uniformly (pruned branches
    stay behind as dead slots). Returns (parents, query_slots, mask) where the mask
    row of a query admits exactly its ancestors and itself.
    """
    steps = (n_kv - 4) // beams
    prefix = n_kv - beams * steps
    if steps < 1 or prefix < 1:
        raise ValueError("tree needs n_kv >= 4 + beams")
    parents = np.full(n_kv, -1, dtype=np.int32)
    parents[1:prefix] = np.arange(prefix - 1)
    prev = np.full(beams, prefix - 1, dtype=np.int32)
    for s in range(steps):
        slots = prefix + beams * s + np.arange(beams, dtype=np.int32)
        src = rng.integers(0, beams, size=beams) if s > 0 else np.zeros(beams, dtype=np.int64)
        parents[slots] = prev[src]
        prev = slots
    query_slots = prev.copy()
    mask = np.zeros((beams, n_kv), dtype=bool)
    for b, slot in enumerate(query_slots):
        node = int(slot)
        while node >= 0:
            mask[b, node] = True
            node = int(parents[node])
    return parents, query_slots, mask


def verify_self_case(trial: int, layer: int, seed: int = 0, n_kv: int | None = None,
                     n_q: int = VERIFY_BLOCK) -> VerifyCase:
    L = cache_length(trial, seed) if n_kv is None else int(n_kv)
    q = normal_f16(rng_for(seed, 4, layer, T_Q, trial), (n_q, N_HEADS, HEAD_DIM), 1.0)
    k = normal_f16(rng_for(seed, 4, layer, T_KSELF, trial), (L, N_HEADS, HEAD_DIM), 1.0)
    v = normal_f16(rng_for(seed, 4, layer, T_VSELF, trial), (L, N_HEADS, HEAD_DIM), 1.0)
    return VerifyCase(q=q, k=k, v=v, mask=causal_block_mask(n_q, L), kind="causal")


def verify_cross_case(trial: int, layer: int, seed: int = 0, n_kv: int = FRAMES_PER_WINDOW,
                      n_q: int = VERIFY_BLOCK) -> VerifyCase:
    q = normal_f16(rng_for(seed, 4, layer, T_Q, trial), (n_q, N_HEADS, HEAD_DIM), 1.0)
    k = normal_f16(rng_for(seed, 4, layer, T_KCROSS, trial), (n_kv, N_HEADS, HEAD_DIM), 1.0)
    v = normal_f16(rng_for(seed, 4, layer, T_VCROSS, trial), (n_kv, N_HEADS, HEAD_DIM), 1.0)
    return VerifyCase(q=q, k=k, v=v, mask=None, kind="cross")


def verify_tree_case(trial: int, layer: int, seed: int = 0, n_kv: int | None = None) -> VerifyCase:
    L = cache_length(trial, seed) if n_kv is None else int(n_kv)
    parents, query_slots, mask = beam_tree(L, rng_for(seed, 4, 0, T_TREE, trial))
    k = normal_f16(rng_for(seed, 4, layer, T_KSELF, trial), (L, N_HEADS, HEAD_DIM), 1.0)
    v = normal_f16(rng_for(seed, 4, layer, T_VSELF, trial), (L, N_HEADS, HEAD_DIM), 1.0)
    # A query's projection is a row of its own slot's input; draw queries independently.
    q = normal_f16(rng_for(seed, 4, layer, T_Q, trial), (BEAMS, N_HEADS, HEAD_DIM), 1.0)
    return VerifyCase(q=q, k=k, v=v, mask=mask, kind="tree", parents=parents, query_slots=query_slots)



# --------------------------------------------------------------------------------------
# The rest of a Whisper-large-v3 encoder around the attention path (pre-norm layer with a
# GELU MLP, convolutional stem, positional embedding, final LayerNorm). Shapes follow the
# public Whisper-large-v3 configuration; the pages give none of these tensors.
# --------------------------------------------------------------------------------------

D_FF = 4 * D_MODEL        # MLP hidden width
N_MELS = 128              # mel bins of the large-v3 front end
MEL_FRAMES = 2 * FRAMES_PER_WINDOW  # 3000 mel frames per 30 s window (conv2 halves them)

(T_LN1G, T_LN1B, T_LN2G, T_LN2B, T_W1, T_B1, T_W2, T_B2, T_BO, T_MEL, T_C1W, T_C1B, T_C2W,
 T_C2B, T_LNPG, T_LNPB) = range(20, 36)

LN_SCALE_VAR = 0.01   # LayerNorm scale 1 + N(0, 0.01); shift N(0, 0.01)


@dataclass
class FullLayerWeights:
    """Math layout (y = x w): w [in, out]."""
    ln1_g: np.ndarray
    ln1_b: np.ndarray
    w_qkv: np.ndarray      # [1280, 3840]
    b_qkv: np.ndarray      # [3840], K third zero
    w_o: np.ndarray        # [1280, 1280]
    b_o: np.ndarray        # [1280]
    ln2_g: np.ndarray
    ln2_b: np.ndarray
    w_fc1: np.ndarray      # [1280, 5120]
    b_fc1: np.ndarray      # [5120]
    w_fc2: np.ndarray      # [5120, 1280]
    b_fc2: np.ndarray      # [1280]


def _ln_params(seed, cfg, layer, tg, tb, d=D_MODEL):
    g = (1.0 + rng_for(seed, cfg, layer, tg).standard_normal(d) * math.sqrt(LN_SCALE_VAR)).astype(np.float16)
    b = normal_f16(rng_for(seed, cfg, layer, tb), (d,), LN_SCALE_VAR)
    return g, b


def full_layer_weights(cfg: int, layer: int, seed: int = 0) -> FullLayerWeights:
    """Attention weights as in encoder_layer_weights (same streams) plus an output bias,
    two LayerNorms and the MLP: W1 ~ N(0, 1/1280), W2 ~ N(0, 1/5120), biases N(0, 0.02)."""
    a = encoder_layer_weights(cfg, layer, seed)
    ln1_g, ln1_b = _ln_params(seed, cfg, layer, T_LN1G, T_LN1B)
    ln2_g, ln2_b = _ln_params(seed, cfg, layer, T_LN2G, T_LN2B)
    return FullLayerWeights(
        ln1_g=ln1_g, ln1_b=ln1_b, w_qkv=a.w_qkv, b_qkv=a.b_qkv, w_o=a.w_o,
        b_o=normal_f16(rng_for(seed, cfg, layer, T_BO), (D_MODEL,), B_VAR),
        ln2_g=ln2_g, ln2_b=ln2_b,
        w_fc1=normal_f16(rng_for(seed, cfg, layer, T_W1), (D_MODEL, D_FF), 1.0 / D_MODEL),
        b_fc1=normal_f16(rng_for(seed, cfg, layer, T_B1), (D_FF,), B_VAR),
        w_fc2=normal_f16(rng_for(seed, cfg, layer, T_W2), (D_FF, D_MODEL), 1.0 / D_FF),
        b_fc2=normal_f16(rng_for(seed, cfg, layer, T_B2), (D_MODEL,), B_VAR))


@dataclass
class StemWeights:
    conv1_w: np.ndarray   # [1280, 128, 3] (out, in, tap)
    conv1_b: np.ndarray   # [1280]
    conv2_w: np.ndarray   # [1280, 1280, 3]
    conv2_b: np.ndarray   # [1280]
    pos_emb: np.ndarray   # [1500, 1280]
    lnp_g: np.ndarray     # final LayerNorm
    lnp_b: np.ndarray


def sinusoidal_positions(length: int, channels: int) -> np.ndarray:
    """Fixed sinusoidal position table [length, channels]: the first half of the channels
    holds sin(t * w_i), the second half cos(t * w_i), with w_i = 10000^(-i / (channels/2 - 1))
    for i = 0 .. channels/2 - 1. Returned in fp16."""
    half = channels // 2
    w = np.exp(-math.log(10000.0) * np.arange(half) / (half - 1))
    t = np.arange(length)[:, None] * w[None, :]
    return np.concatenate([np.sin(t), np.cos(t)], axis=1).astype(np.float16)


def stem_weights(cfg: int = 1, seed: int = 0, frames: int = FRAMES_PER_WINDOW) -> StemWeights:
    """conv1 ~ N(0, 1/384) (fan-in 3 * 128), conv2 ~ N(0, 1/3840), biases N(0, 0.02)."""
    lnp_g, lnp_b = _ln_params(seed, cfg, 0, T_LNPG, T_LNPB)
    return StemWeights(
        conv1_w=normal_f16(rng_for(seed, cfg, 0, T_C1W), (D_MODEL, N_MELS, 3), 1.0 / (3 * N_MELS)),
        conv1_b=normal_f16(rng_for(seed, cfg, 0, T_C1B), (D_MODEL,), B_VAR),
        conv2_w=normal_f16(rng_for(seed, cfg, 0, T_C2W), (D_MODEL, D_MODEL, 3), 1.0 / (3 * D_MODEL)),
        conv2_b=normal_f16(rng_for(seed, cfg, 0, T_C2B), (D_MODEL,), B_VAR),
        pos_emb=sinusoidal_positions(frames, D_MODEL), lnp_g=lnp_g, lnp_b=lnp_b)


def mel_input(batch: int = 1, cfg: int = 1, seed: int = 0, frames: int = MEL_FRAMES) -> np.ndarray:
    """Synthetic log-mel input [batch, 128, frames] ~ N(0, 1), fp16 (channel-major per window)."""
    return normal_f16(rng_for(seed, cfg, 0, T_MEL), (batch, N_MELS, frames), 1.0)


# --------------------------------------------------------------------------------------
# The decoder's verification layer (self-attention over the KV cache, cross-attention over
# the encoder output, MLP), Whisper-large-v3 decoder geometry (same width and heads).
# --------------------------------------------------------------------------------------

(T_DLN1G, T_DLN1B, T_DLN2G, T_DLN2B, T_DLN3G, T_DLN3B, T_DWQKV, T_DBQ, T_DBV, T_DWO, T_DBO, T_DWQC, T_DBQC,
 T_DWOC, T_DBOC, T_DWCK, T_DWCV, T_DBCV, T_DW1, T_DB1, T_DW2, T_DB2, T_DX) = range(40, 63)


@dataclass
class DecoderLayerWeights:
    """Math layout (y = x w): w [in, out]."""
    ln1_g: np.ndarray
    ln1_b: np.ndarray
    w_qkv: np.ndarray      # [1280, 3840], K third of b_qkv zero
    b_qkv: np.ndarray
    w_o: np.ndarray
    b_o: np.ndarray
    ln2_g: np.ndarray
    ln2_b: np.ndarray
    w_qc: np.ndarray       # cross-attention query projection [1280, 1280]
    b_qc: np.ndarray
    w_oc: np.ndarray
    b_oc: np.ndarray
    w_ck: np.ndarray       # cross-attention key / value projections of the encoder output
    w_cv: np.ndarray
    b_cv: np.ndarray
    ln3_g: np.ndarray
    ln3_b: np.ndarray
    w_fc1: np.ndarray
    b_fc1: np.ndarray
    w_fc2: np.ndarray
    b_fc2: np.ndarray


def decoder_layer_weights(layer: int, seed: int = 0, cfg: int = 4) -> DecoderLayerWeights:
    """Distributions as for the encoder layer: matrices N(0, 1/fan-in), biases N(0, 0.02),
    LayerNorm scale 1 + N(0, 0.01) and shift N(0, 0.01); no key biases."""
    g = lambda tid, shape, var: normal_f16(rng_for(seed, cfg, layer, tid), shape, var)
    ln = lambda tg, tb: _ln_params(seed, cfg, layer, tg, tb)
    ln1_g, ln1_b = ln(T_DLN1G, T_DLN1B)
    ln2_g, ln2_b = ln(T_DLN2G, T_DLN2B)
    ln3_g, ln3_b = ln(T_DLN3G, T_DLN3B)
    b_qkv = np.zeros(QKV_COLS, dtype=np.float16)
    b_qkv[:D_MODEL] = g(T_DBQ, (D_MODEL,), B_VAR)
    b_qkv[2 * D_MODEL:] = g(T_DBV, (D_MODEL,), B_VAR)
    return DecoderLayerWeights(
        ln1_g=ln1_g, ln1_b=ln1_b, w_qkv=g(T_DWQKV, (D_MODEL, QKV_COLS), W_VAR), b_qkv=b_qkv,
        w_o=g(T_DWO, (D_MODEL, D_MODEL), W_VAR), b_o=g(T_DBO, (D_MODEL,), B_VAR),
        ln2_g=ln2_g, ln2_b=ln2_b, w_qc=g(T_DWQC, (D_MODEL, D_MODEL), W_VAR), b_qc=g(T_DBQC, (D_MODEL,), B_VAR),
        w_oc=g(T_DWOC, (D_MODEL, D_MODEL), W_VAR), b_oc=g(T_DBOC, (D_MODEL,), B_VAR),
        w_ck=g(T_DWCK, (D_MODEL, D_MODEL), W_VAR), w_cv=g(T_DWCV, (D_MODEL, D_MODEL), W_VAR),
        b_cv=g(T_DBCV, (D_MODEL,), B_VAR),
        ln3_g=ln3_g, ln3_b=ln3_b, w_fc1=g(T_DW1, (D_MODEL, D_FF), 1.0 / D_MODEL), b_fc1=g(T_DB1, (D_FF,), B_VAR),
        w_fc2=g(T_DW2, (D_FF, D_MODEL), 1.0 / D_FF), b_fc2=g(T_DB2, (D_MODEL,), B_VAR))


def decoder_block_input(trial: int = 0, n_q: int = VERIFY_BLOCK, seed: int = 0, cfg: int = 4) -> np.ndarray:
    """Residual-stream rows of the n_q block tokens [n_q, 1280] ~ N(0, 1)."""
    return normal_f16(rng_for(seed, cfg, 0, T_DX, trial), (n_q, D_MODEL), 1.0)


# --------------------------------------------------------------------------------------
# Packed QKV buffers with planted scores (online-softmax edge cases).
# --------------------------------------------------------------------------------------

PLANT_KEY_VALUE = 4.0   # the one non-zero coordinate of a planted key
PLANT_COORDS = 8        # coordinates 0..7 of every head are reserved for planting


@dataclass
class Plant:
    """Query rows `rows` (window-local) of window `window` hold a * e_c in every head and the
    key at window-local position `key` holds PLANT_KEY_VALUE * e_c; c = `coord` (< 8).  With
    the reserved coordinates of every other key zero, these rows score 0 against every other
    key and a * PLANT_KEY_VALUE / 8 against the planted one."""
    coord: int
    a: float
    key: int
    rows: list
    window: int = 0


def plant_scale(excess_log2: float) -> float:
    """Query amplitude a whose score against a planted key is `excess_log2` in log2 units
    (a * PLANT_KEY_VALUE / 8 * log2(e) = excess)."""
    return float(excess_log2) * 8.0 / (PLANT_KEY_VALUE * math.log2(math.e))


def planted_qkv(batch: int, seq_len: int, plants, seed: int = 0) -> np.ndarray:
    """fp16 [batch*seq_len, 3840] packed Q | K | V drawn N(0, 1), with the reserved key
    coordinates zeroed and the plants written in (all 20 heads alike)."""
    r = rng_for(seed, 90, 0, T_X)
    qkv = r.standard_normal((batch * seq_len, QKV_COLS)).astype(np.float16)
    q = qkv[:, :D_MODEL].reshape(-1, N_HEADS, HEAD_DIM)
    k = qkv[:, D_MODEL:2 * D_MODEL].reshape(-1, N_HEADS, HEAD_DIM)
    k[:, :, :PLANT_COORDS] = 0
    for p in plants:
        base = p.window * seq_len
        for row in p.rows:
            q[base + row] = 0
            q[base + row, :, p.coord] = np.float16(p.a)
        k[base + p.key] = 0
        k[base + p.key, :, p.coord] = np.float16(PLANT_KEY_VALUE)
    return qkv
