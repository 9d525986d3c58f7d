"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

This module only draws random numbers; it holds none of the training step's
arithmetic.  It stands in for the FineWeb token shards that the pretraining
paper trains on (Pretraining and adapting a language model on a
dependency-free stack, §4.2 corpus preparation), which are not available here.

Token stream (all configurations): the stream opens with an end-of-text id,
then repeats {a document of length l ~ Geometric(p=1/40) on {1, 2, ...}, its
tokens i.i.d. from a finite Zipf(s=1.1) law over the ids 0..V-2, then the
end-of-text id V-1}.  Each document is therefore preceded by an end-of-text
marker, as the paper's corpus preparation does.  Micro-step k of a run takes
B*T+1 consecutive stream tokens starting at k*B*T; row b's inputs are
buf[b*T:(b+1)*T] and its targets are buf[b*T+1:(b+1)*T+1].
"""
from __future__ import annotations

import numpy as np

DEFAULT_SEED = 1337
ZIPF_S = 1.1
DOC_P = 1.0 / 40.0

# Independent child streams of SeedSequence(seed): one per purpose.
STREAM_TOKENS = 0
STREAM_TENSORS = 1


def child_rng(seed: int, stream: int) -> np.random.Generator:
    """Generator for one purpose, spawned from SeedSequence(seed)."""
    return np.random.default_rng(np.random.SeedSequence(seed).spawn(stream + 1)[stream])


def zipf_cdf(n_ids: int, s: float = ZIPF_S) -> np.ndarray:
    """CDF of the finite Zipf law P(r) proportional to (r+1)^-s over r in [0, n_ids)."""
    w = np.arange(1, n_ids + 1, dtype=np.float64) ** (-s)
    c = np.cumsum(w)
    return c / c[-1]


def token_stream(n_tokens: int, V: int, seed: int = DEFAULT_SEED, stream: int = STREAM_TOKENS) -> np.ndarray:
    """Return n_tokens int32 ids of the Zipf/EOT stream described in the module docstring."""
    rng = child_rng(seed, stream)
    eot = V - 1
    cdf = zipf_cdf(V - 1)
    out = np.empty(0, dtype=np.int32)
    while out.size < n_tokens:
        need = n_tokens - out.size
        n_docs = max(16, int(need * DOC_P * 1.25) + 16)
        lens = rng.geometric(DOC_P, size=n_docs).astype(np.int64)
        total = int(lens.sum()) + n_docs
        body = np.searchsorted(cdf, rng.random(total - n_docs), side="right").astype(np.int32)
        np.minimum(body, V - 2, out=body)
        chunk = np.empty(total, dtype=np.int32)
        starts = np.concatenate(([0], np.cumsum(lens + 1)[:-1]))
        is_eot = np.zeros(total, dtype=bool)
        is_eot[starts] = True
        chunk[is_eot] = eot
        chunk[~is_eot] = body
        out = np.concatenate((out, chunk))
    return out[:n_tokens]


def micro_batches(n_micro: int, B: int, T: int, V: int, seed: int = DEFAULT_SEED):
    """List of (tok, tgt) int32 [B, T] pairs for n_micro consecutive micro-steps."""
    BT = B * T
    buf = token_stream(n_micro * BT + 1, V, seed)
    res = []
    for k in range(n_micro):
        chunk = buf[k * BT: k * BT + BT + 1]
        tok = chunk[:BT].reshape(B, T).copy()
        tgt = chunk[1:BT + 1].reshape(B, T).copy()
        res.append((tok, tgt))
    return res


def normal(shape, std: float = 1.0, seed: int = DEFAULT_SEED, stream: int = STREAM_TENSORS,
           dtype=np.float32) -> np.ndarray:
    """Seeded N(0, std^2) array (used for kernel-level inputs: logits, activations, grads)."""
    rng = child_rng(seed, stream)
    return (rng.standard_normal(size=shape) * std).astype(dtype)


def targets(rows: int, V: int, seed: int = DEFAULT_SEED) -> np.ndarray:
    """Targets for kernel-level loss inputs: the first `rows` ids of the token stream shifted by one."""
    return token_stream(rows + 1, V, seed)[1:].astype(np.int32)


class TokenStream:
    """Resumable stream of the same Zipf/EOT law as token_stream (a different draw
    order, so not the same ids for a seed).  Documents are drawn 64 at a time;
    state() captures the generator state and the unread tokens, and
    TokenStream.from_state() continues exactly where state() was taken."""

    DOCS_PER_DRAW = 64

    def __init__(self, V: int, seed: int = DEFAULT_SEED, stream: int = STREAM_TOKENS):
        self.V = V
        self.rng = child_rng(seed, stream)
        self.cdf = zipf_cdf(V - 1)
        self.buf = np.empty(0, dtype=np.int32)

    def _draw(self):
        V, n = self.V, self.DOCS_PER_DRAW
        lens = self.rng.geometric(DOC_P, size=n).astype(np.int64)
        body = np.searchsorted(self.cdf, self.rng.random(int(lens.sum())), side="right").astype(np.int32)
        np.minimum(body, V - 2, out=body)
        chunk = np.empty(int(lens.sum()) + n, dtype=np.int32)
        starts = np.concatenate(([0], np.cumsum(lens + 1)[:-1]))
        is_eot = np.zeros(chunk.size, dtype=bool)
        is_eot[starts] = True
        chunk[is_eot] = V - 1
        chunk[~is_eot] = body
        self.buf = np.concatenate((self.buf, chunk))

    def take(self, n: int, keep_last: bool = False) -> np.ndarray:
        """The next n ids; with keep_last the n-th id is also the first of the next take."""
        while self.buf.size < n:
            self._draw()
        out = self.buf[:n].copy()
        self.buf = self.buf[n - 1 if keep_last else n:]
        return out

    def state(self) -> dict:
        return {"V": self.V, "rng": self.rng.bit_generator.state, "buf": self.buf.tolist()}

    @classmethod
    def from_state(cls, st: dict) -> "TokenStream":
        obj = cls.__new__(cls)
        obj.V = int(st["V"])
        obj.rng = np.random.default_rng()
        obj.rng.bit_generator.state = st["rng"]
        obj.cdf = zipf_cdf(obj.V - 1)
        obj.buf = np.asarray(st["buf"], dtype=np.int32)
        return obj

    def micro_batch(self, B: int, T: int):
        """(tok, tgt) int32 [B, T] from the next B*T+1 ids (consecutive micro-batches share one id)."""
        chunk = self.take(B * T + 1, keep_last=True)
        return chunk[:-1].reshape(B, T).copy(), chunk[1:].reshape(B, T).copy()
