"""Seeded synthetic workloads for the causal long convolution.

This module only *generates inputs*; it holds none of the convolution's
arithmetic.  Both the GPU library's tests/benchmark and the CPU oracle read
their inputs from here, so the two sides always see identical values.

Every row is generated from its own counter-seeded numpy stream
(``numpy.random.default_rng([231105908, workload_id, stream, index])``), so
any subset of rows (or kernel channels) can be produced on its own and is
bit-identical to the same rows of the full tensor.  Values are drawn in fp64
and rounded to nearest-even to the storage dtype (u: the I/O dtype; k: fp32).

Workload shapes follow the sizes the FlashFFTConv page benchmarks (batch 64,
hidden 768, lengths from 256 up to 4M; section 5) and the application
lengths it names (64 kHz raw audio, ~2.3 Mbp genes; section 2).  Actual model
activations, audio clips and genomes are not available, so seeded synthetic
stand-ins of the same shape and value structure are used instead.

bf16 data is carried as ``uint16`` bit patterns (numpy has no bf16 dtype).
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

SEED = 231105908


@dataclass(frozen=True)
class Workload:
    name: str
    wid: int            # seed component, one per workload
    B: int
    H: int
    N: int
    dtype: str          # I/O dtype of u and y: 'f32', 'f16' or 'bf16'
    u_kind: str         # 'normal' | 'sines' | 'onehot'
    k_kind: str         # 'normal_scaled' | 'decay'
    desc: str

    @property
    def rows(self) -> int:
        return self.B * self.H


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_f32_n256", 1, 1, 4, 256, "f32", "normal",
                 "normal_scaled",
                 "u ~ N(0,1); k ~ N(0,1)/sqrt(N); fp32 in and out"),
        Workload("hyena_bf16_n1k", 2, 64, 768, 1024, "bf16", "normal",
                 "decay",
                 "Hyena-style: u ~ N(0,1) in bf16; k = N(0,1)*exp(-a_h t)"),
        Workload("m2bert_f16_n8k", 3, 16, 768, 8192, "f16", "normal",
                 "decay",
                 "M2-BERT/Hyena long context: u ~ N(0,1) in fp16"),
        Workload("longconv_bf16_n32k", 6, 4, 512, 32768, "bf16", "normal",
                 "decay",
                 "32K-sample long convolution, the longest length the page "
                 "runs fully fused: u ~ N(0,1) in bf16"),
        Workload("audio_bf16_n64k", 4, 4, 256, 65536, "bf16", "sines",
                 "decay",
                 "raw-audio shaped: 8 random tones at 64 kHz + 0.1 N(0,1)"),
        Workload("genome_bf16_n4m", 5, 1, 128, 4194304, "bf16", "onehot",
                 "decay",
                 "genome scale: one-hot over 4 channel groups for the first "
                 "2.3M positions, zero after"),
    ]
}

GENOME_LEN = 2_300_000      # one-hot region of the genome workload
AUDIO_RATE = 64000.0        # samples per second of the audio workload


def _rng(wid: int, stream: int, index: int = 0) -> np.random.Generator:
    return np.random.default_rng([SEED, wid, stream, index])


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even); return uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (b >> 16) & 1
    return ((b + 0x7FFF + lsb) >> 16).astype(np.uint16)


def cast_io(x64: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 -> storage dtype (RNE).  bf16 goes through fp32 first."""
    if dtype == "f32":
        return x64.astype(np.float32)
    if dtype == "f16":
        return x64.astype(np.float16)
    if dtype == "bf16":
        return f32_to_bf16_bits(x64.astype(np.float32))
    raise ValueError(dtype)


def decay_rates(w: Workload) -> np.ndarray:
    """a_h, log-uniform in [1e-3, 1e-1], one per channel."""
    return 10.0 ** _rng(w.wid, 2).uniform(-3.0, -1.0, size=w.H)


def kernel_rows(w: Workload, hs=None) -> np.ndarray:
    """Convolution kernel rows k[h, 0:N] as fp32, shape [len(hs), N]."""
    hs = np.arange(w.H) if hs is None else np.asarray(hs, dtype=np.int64)
    out = np.empty((len(hs), w.N), dtype=np.float32)
    t = np.arange(w.N, dtype=np.float64)
    a = decay_rates(w) if w.k_kind == "decay" else None
    for i, h in enumerate(hs):
        g = _rng(w.wid, 1, int(h)).standard_normal(w.N)
        if w.k_kind == "normal_scaled":
            row = g / np.sqrt(w.N)
        elif w.k_kind == "decay":
            row = g * np.exp(-a[h] * t)
        else:
            raise ValueError(w.k_kind)
        out[i] = row.astype(np.float32)
    return out


def _genome_symbols(w: Workload) -> np.ndarray:
    return _rng(w.wid, 3).integers(0, 4, size=GENOME_LEN)


def input_rows(w: Workload, rows=None) -> np.ndarray:
    """Input rows u[r, 0:N] (r = b*H + h) in the storage dtype."""
    rows = np.arange(w.rows) if rows is None else np.asarray(rows, np.int64)
    if w.dtype == "f32":
        out = np.empty((len(rows), w.N), dtype=np.float32)
    elif w.dtype == "f16":
        out = np.empty((len(rows), w.N), dtype=np.float16)
    else:
        out = np.empty((len(rows), w.N), dtype=np.uint16)
    sym = _genome_symbols(w) if w.u_kind == "onehot" else None
    t = np.arange(w.N, dtype=np.float64)
    for i, r in enumerate(rows):
        r = int(r)
        if w.u_kind == "normal":
            x = _rng(w.wid, 0, r).standard_normal(w.N)
        elif w.u_kind == "sines":
            g = _rng(w.wid, 0, r)
            amp = g.uniform(0.1, 1.0, size=8)
            freq = 10.0 ** g.uniform(np.log10(20.0), np.log10(20000.0), 8)
            phase = g.uniform(0.0, 2.0 * np.pi, size=8)
            x = 0.1 * g.standard_normal(w.N)
            for j in range(8):
                x += amp[j] * np.sin(2.0 * np.pi * freq[j] * t / AUDIO_RATE
                                     + phase[j])
        elif w.u_kind == "onehot":
            h = r % w.H
            x = np.zeros(w.N)
            n = min(w.N, GENOME_LEN)
            x[:n] = (sym[:n] == (h // 32)).astype(np.float64)
        else:
            raise ValueError(w.u_kind)
        out[i] = cast_io(x, w.dtype)
    return out


def gate_rows(w: Workload, which: str, rows=None) -> np.ndarray:
    """Gate rows of the gated convolution (r = b*H + h) in the storage
    dtype: which = "w" (input gate) or "v" (output gate), each N(0,1) --
    in H3/Hyena-style layers both gates are linear projections of the
    layer input, Gaussian-like at initialisation."""
    stream = {"w": 4, "v": 5, "dy": 6}[which]
    rows = np.arange(w.rows) if rows is None else np.asarray(rows, np.int64)
    dt = {"f32": np.float32, "f16": np.float16, "bf16": np.uint16}[w.dtype]
    out = np.empty((len(rows), w.N), dtype=dt)
    for i, r in enumerate(rows):
        out[i] = cast_io(_rng(w.wid, stream, int(r)).standard_normal(w.N),
                         w.dtype)
    return out


def dy_rows(w: Workload, rows=None) -> np.ndarray:
    """Output-gradient rows dL/dy for the backward pass (r = b*H + h), N(0,1)
    in the storage dtype (a loss with Gaussian sensitivities)."""
    return gate_rows(w, "dy", rows)


def shrink(w: Workload, B: int | None = None, H: int | None = None,
           N: int | None = None) -> Workload:
    """Same generator recipe at a smaller shape (parity cases that the
    oracle finishes quickly).  Rows of the shrunk workload with the same
    (b, h) and N are identical to the full workload's rows only when H and
    N are unchanged."""
    from dataclasses import replace
    return replace(w, B=B or w.B, H=H or w.H, N=N or w.N)
