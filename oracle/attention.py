"""fp64 CPU oracle for encoder and verification attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or link
this module: only the tests, the smoke check and the benchmark's CPU-baseline
leg use it. It shares no code with the HIP library (no kernels, headers,
helpers, constants or pre/post-processing); it reads the same fp16 inputs,
upcast exactly to float64, and computes the plain definition with no rounding
of intermediates and no blocking, fusion or reordering.

What it computes, and the passages it follows:

* Packed QKV projection, then attention, then the output projection:
  "audio.cpp PR #1223, Add Edda ASR" — PR description (the encoder projects
  Q, K and V in one packed GEMM and runs flash attention with fp16 keys and
  values) and the encoder commit message (the shared encoder materializes F32
  scores for all 1500 frames; packing QKV and flash attention give the same
  transcripts faster). Flash attention is an exact
  reordering of softmax attention, so the oracle is softmax attention written
  out: full score matrix, masked softmax, P·V, output projection. The attention
  call taking the output projection and the score scale together follows the
  llama.cpp DSpark diff, src/models/dflash.cpp ("cache-aware, non-causal
  attention" hunk).
* Bidirectional encoder (no causal mask): "BuzzASR/danish discussion #1",
  first reply (every encoder position attends to every other one).
* Chunk-local attention: "higgs-audio-v3-stt-GGUF" model card, "Architecture
  note (chunked encoder)": 4 s chunks encoded independently with within-chunk
  attention; a valid frame must not attend to padding.
* Block verification: "audio.cpp PR #1223" — the target verifies the anchor
  plus up to 15 drafted tokens in one pass with KV slots indexed by position;
  beam search shares one token-tree KV cache whose mask row for a beam admits
  only its ancestors.

Readings taken where the pages are silent (each listed in the design notes):
heads are contiguous 64-column slices of each Q|K|V third; the score scale is
1/sqrt(head_dim); a key j is admitted for query row i of a window iff
lo_i <= j < hi_i with lo_i = c*floor(i/c) (0 when c = 0) and
hi_i = min(lo_i + c, valid_len) (valid_len when c = 0); a query row with no
admitted key yields a zero output; "ancestors" includes the node itself.

Parity pins: every function here is pinned in tests/test_oracle.py by brute
force on tiny shapes, closed forms, invariants and an independent library
routine (torch scaled_dot_product_attention in float64 on the CPU).
"""
from __future__ import annotations

import math

import numpy as np


def as_f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


# ---------------------------------------------------------------------------
# Step 1: packed projection.
# ---------------------------------------------------------------------------

def qkv_projection(x, w_qkv, b_qkv=None) -> np.ndarray:
    """QKV = X W_qkv + b_qkv in float64. X [rows, d], W_qkv [d, 3d] with column
    blocks Q | K | V. Returns [rows, 3d]."""
    out = as_f64(x) @ as_f64(w_qkv)
    if b_qkv is not None:
        out = out + as_f64(b_qkv)[None, :]
    return out


def split_heads(block, n_heads: int) -> np.ndarray:
    """[rows, n_heads*dh] -> [n_heads, rows, dh]; head h owns columns dh*h .. dh*h+dh-1."""
    rows, width = block.shape
    dh = width // n_heads
    return block.reshape(rows, n_heads, dh).transpose(1, 0, 2)


# ---------------------------------------------------------------------------
# Step 2: which keys a query row admits.
# ---------------------------------------------------------------------------

def key_interval(i: int, chunk_len: int, valid_len: int) -> tuple[int, int]:
    """Admitted key interval [lo, hi) of query row i inside one window.

    chunk_len == 0: the whole window up to valid_len (bidirectional encoder).
    chunk_len  > 0: only the row's own chunk, cut at valid_len (padding keys are
    never attended to)."""
    if chunk_len == 0:
        return 0, int(valid_len)
    lo = chunk_len * (i // chunk_len)
    return lo, min(lo + chunk_len, int(valid_len))


def encoder_admit_mask(seq_len: int, chunk_len: int, valid_len: int) -> np.ndarray:
    """bool [seq_len, seq_len]: entry (i, j) is True iff query row i admits key j."""
    admit = np.zeros((seq_len, seq_len), dtype=bool)
    for i in range(seq_len):
        lo, hi = key_interval(i, chunk_len, valid_len)
        if hi > lo:
            admit[i, lo:hi] = True
    return admit


def causal_rows(n_q: int, n_kv: int) -> np.ndarray:
    """Causal mask rows for a block of n_q tokens occupying the last n_q KV slots
    (slot = position): query t admits keys 0 .. n_kv - n_q + t."""
    admit = np.zeros((n_q, n_kv), dtype=bool)
    for t in range(n_q):
        admit[t, : n_kv - n_q + t + 1] = True
    return admit


# ---------------------------------------------------------------------------
# Steps 3-5: masked softmax attention for one head.
# ---------------------------------------------------------------------------

def softmax_probabilities(q, k, admit, scale: float) -> np.ndarray:
    """P [n_q, n_kv]: P_ij = exp(s_ij - max_j s_ij) / sum_j exp(s_ij - max_j s_ij) over the
    admitted keys, s_ij = scale * (q_i . k_j); P_ij = 0 on masked keys and on rows with
    no admitted key."""
    s = (as_f64(q) @ as_f64(k).T) * scale
    s = np.where(admit, s, -np.inf)
    p = np.zeros_like(s)
    live = admit.any(axis=1)
    if live.any():
        sl = s[live]
        m = sl.max(axis=1, keepdims=True)
        e = np.exp(sl - m)
        p[live] = e / e.sum(axis=1, keepdims=True)
    return p


def attention_head(q, k, v, admit, scale: float) -> np.ndarray:
    """O = P V for one head. q [n_q, dh], k/v [n_kv, dh], admit bool [n_q, n_kv]."""
    return softmax_probabilities(q, k, admit, scale) @ as_f64(v)


# ---------------------------------------------------------------------------
# Encoder attention sublayer: projection -> attention -> output projection.
# ---------------------------------------------------------------------------

def encoder_attention(x, w_qkv, b_qkv, w_o, b_o, batch: int, seq_len: int, chunk_len: int,
                      valid_len, n_heads: int, rows=None, head_dim: int | None = None) -> dict:
    """One encoder attention sublayer over `batch` windows of `seq_len` rows.

    x [batch*seq_len, d]; w_qkv [d, 3d]; b_qkv [3d] or None; w_o [d, d]; b_o [d] or None;
    valid_len: int per window (keys at positions >= valid_len are masked; every query
    row is still computed). `rows`: optional sorted array of global row indices to
    compute outputs for (every key of their windows is still projected); default all.

    Returns float64 arrays {"qkv": [rows_sel, 3d] (the selected rows' projection),
    "o": [rows_sel, d] (heads concatenated), "y": [rows_sel, d]} and "rows".
    """
    x = as_f64(x)
    d = x.shape[1]
    dh = d // n_heads if head_dim is None else head_dim
    scale = 1.0 / math.sqrt(dh)
    valid_len = np.broadcast_to(np.asarray(valid_len, dtype=np.int64), (batch,))
    rows = np.arange(batch * seq_len) if rows is None else np.asarray(rows, dtype=np.int64)
    qkv_sel = np.zeros((rows.size, 3 * d))
    o_sel = np.zeros((rows.size, d))
    for b in range(batch):
        pick = np.nonzero((rows >= b * seq_len) & (rows < (b + 1) * seq_len))[0]
        if pick.size == 0:
            continue
        local = rows[pick] - b * seq_len
        qkv = qkv_projection(x[b * seq_len:(b + 1) * seq_len], w_qkv, b_qkv)
        qkv_sel[pick] = qkv[local]
        q = split_heads(qkv[local, :d], n_heads)
        k = split_heads(qkv[:, d:2 * d], n_heads)
        v = split_heads(qkv[:, 2 * d:], n_heads)
        admit = encoder_admit_mask(seq_len, chunk_len, int(valid_len[b]))[local]
        for h in range(n_heads):
            o_sel[pick, h * dh:(h + 1) * dh] = attention_head(q[h], k[h], v[h], admit, scale)
    y = o_sel @ as_f64(w_o)
    if b_o is not None:
        y = y + as_f64(b_o)[None, :]
    return {"qkv": qkv_sel, "o": o_sel, "y": y, "rows": rows}


# ---------------------------------------------------------------------------
# Verification attention: n_q block queries against a KV cache, per head.
# ---------------------------------------------------------------------------

def verify_attention(q, k, v, mask=None) -> np.ndarray:
    """O [n_q, H, dh] = softmax over admitted cache slots of (q.k / sqrt(dh)), times V.

    q [n_q, H, dh]; k, v [n_kv, H, dh] (row = slot = position); mask bool [n_q, n_kv]
    (True = admitted) or None (every slot admitted, e.g. cross-attention)."""
    q, k, v = as_f64(q), as_f64(k), as_f64(v)
    n_q, n_heads, dh = q.shape
    admit = np.ones((n_q, k.shape[0]), dtype=bool) if mask is None else np.asarray(mask, dtype=bool)
    out = np.zeros((n_q, n_heads, dh))
    for h in range(n_heads):
        out[:, h, :] = attention_head(q[:, h, :], k[:, h, :], v[:, h, :], admit, 1.0 / math.sqrt(dh))
    return out


def partial_attention(q, k, v, admit, scale: float):
    """Softmax statistics of one subset of keys for one head: (m, l, o) with
    m_i = max admitted score, l_i = sum exp(s - m_i), o_i = sum exp(s - m_i) v (unnormalized).
    A row with no admitted key in the subset has m = -inf, l = 0, o = 0."""
    s = np.where(admit, (as_f64(q) @ as_f64(k).T) * scale, -np.inf)
    n_q = s.shape[0]
    m = np.full(n_q, -np.inf)
    l = np.zeros(n_q)
    o = np.zeros((n_q, np.shape(v)[1]))
    for i in range(n_q):
        if admit[i].any():
            m[i] = s[i].max()
            e = np.exp(s[i] - m[i])
            l[i] = e.sum()
            o[i] = e @ as_f64(v)
    return m, l, o


def merge_partials(parts) -> np.ndarray:
    """Combine (m, l, o) partials of disjoint key subsets into the softmax output:
    m = max_s m_s, l = sum_s l_s e^(m_s - m), O = sum_s o_s e^(m_s - m) / l (O = 0 when l = 0)."""
    ms = np.stack([p[0] for p in parts])          # [S, n_q]
    m = ms.max(axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(ms), np.exp(ms - safe_m[None, :]), 0.0)
    l = sum(w[s] * parts[s][1] for s in range(len(parts)))
    o = sum(w[s][:, None] * parts[s][2] for s in range(len(parts)))
    out = np.zeros_like(o)
    nz = l > 0
    out[nz] = o[nz] / l[nz][:, None]
    return out


# ---------------------------------------------------------------------------
# Work accounting (algorithmic FLOPs), for reporting only.
# ---------------------------------------------------------------------------

def admitted_pairs(seq_len: int, chunk_len: int, valid_len: int) -> int:
    return int(sum(max(0, hi - lo) for lo, hi in (key_interval(i, chunk_len, valid_len)
                                                  for i in range(seq_len))))
