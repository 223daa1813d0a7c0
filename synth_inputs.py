"""Seeded synthetic inputs for the GEMM -> residual -> RMSNorm -> GEMM(+SwiGLU) chain.

This module is the ONLY code shared by the fp64 oracle (``oracle/``) and the HIP path
(``gemm_epilogue_transformer_amd/``).  It draws random numbers and stores them in the
chain's input dtypes; it holds none of the chain's arithmetic (no GEMM, no residual,
no RMSNorm, no gamma fold, no quantisation, no activation).

Workloads.  The pages evaluate LLaMA-style Transformer blocks at 16K-token batches
(ecosistemastartup "CODA: Nuevo kernel GPU..." section "Que mejoras de rendimiento
reporta el paper?"; kucoin "CODA: new research..." section "Resultados del
experimento", hidden dims of 1B/7B/70B models).  No dataset or trained weights are
involved: every tensor here is synthetic with the shapes of those blocks.

Distributions (the same for every workload):
  activations A ~ N(0, 1), residual x_res ~ N(0, 1),
  weights W ~ N(0, 1/K) (variance 1/K, K = that weight's reduction dim),
  gamma = 1 + 0.1 * N(0, 1) (fp32).
All samples are drawn in fp32 from numpy's PCG64 ``default_rng(seed)`` in the fixed
order A, Wo, x_res, gamma, W, then rounded to bf16 (round-to-nearest-even, done by
torch's CPU dtype cast, a library routine).

Weights are stored K-contiguous, i.e. in the [out_features, in_features] layout of
``torch.nn.Linear``: the mathematical Wo[K1, d] is held as Wo_t[d, K1] and the
mathematical Wgu[d, 2F] as W_t[2F, d] (gate rows first, then up rows).
"""

from __future__ import annotations

import dataclasses

import numpy as np

ACT_NONE = 0
ACT_SWIGLU = 1
ACT_ROPE = 2      # rotary position embedding on the QKV product (no activation)
ACT_CE = 3        # cross-entropy of the LM-head product against per-row targets
ACT_SWIGLU_BWD = 4  # backward of the RMSNorm -> GEMM -> SwiGLU block (no first GEMM)
ACT_CHAIN_BWD = 5   # backward of the whole chain (first GEMM + residual included)
ACT_ROPE_BWD = 6    # backward of the RMSNorm -> QKV GEMM -> RoPE block (no first GEMM)
ACT_CE_BWD = 7      # backward of the RMSNorm -> LM head -> cross-entropy block (no first GEMM)


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    M: int          # tokens (rows)
    K1: int         # reduction dim of the first GEMM
    d: int          # hidden dim = N of the first GEMM = reduction dim of the second GEMM
    N2w: int        # rows of the second weight (2F for SwiGLU, N2 otherwise)
    act: int        # ACT_NONE, ACT_SWIGLU, ACT_ROPE or ACT_CE (then N2w = vocabulary size)
    dtype: str      # "bf16" or "e4m3" (fp8 variant: A, Wo and the second weight in e4m3)
    eps: float
    seed: int
    # RoPE only: the first rot_cols output columns are Q and K heads of head_dim values,
    # the tokens are M / seq_len sequences of seq_len positions, base of the angles
    rot_cols: int = 0
    head_dim: int = 64
    seq_len: int = 0
    rope_base: float = 500000.0

    @property
    def n_out(self) -> int:
        return self.N2w // 2 if self.act == ACT_SWIGLU else self.N2w

    @property
    def gemm_flops(self) -> int:
        """2*M*K*N for each of the two GEMMs (epilogue arithmetic not counted); for the
        backward workload the recomputed forward product, the input-gradient product and
        the weight-gradient product (all three of shape M x d x 2F)."""
        if self.act == ACT_SWIGLU_BWD:
            return 3 * (2 * self.M * self.d * self.N2w)
        if self.act == ACT_CHAIN_BWD:
            # plus the first GEMM's input-gradient and weight-gradient products
            return 3 * (2 * self.M * self.d * self.N2w) + 2 * (2 * self.M * self.K1 * self.d)
        if self.act == ACT_CE_BWD:
            # the recomputed logits product, the input-gradient and weight-gradient products
            return 3 * (2 * self.M * self.d * self.N2w)
        if self.act == ACT_ROPE_BWD:
            # the input-gradient and weight-gradient products (the rotation needs no
            # recomputed forward product)
            return 2 * (2 * self.M * self.d * self.N2w)
        return 2 * self.M * self.K1 * self.d + 2 * self.M * self.d * self.N2w


# The five workloads.  1: tiny correctness case; 2: LLaMA-3-1B attention-out ->
# SwiGLU MLP-in; 3: LLaMA-3-1B MLP-out -> next layer QKV (32x64 query + 2x8x64 KV
# heads = 3072); 4: LLaMA-3-8B-shaped attention-out -> SwiGLU MLP-in; 5: workload 2
# with A, Wo and the second weight quantised to e4m3 (same draws as workload 2);
# 6: workload 3 with RoPE on its Q and K columns (32 + 8 heads of 64 = 2560 of the 3072
# columns; V passes), 16384 tokens = 4 sequences of 4096 (same draws as workload 3);
# 7: the last block of LLaMA-3-1B -- MLP-out + residual, final RMSNorm, LM head over the
# 128256-token vocabulary -- ending in the cross-entropy loss against uniform targets;
# 8: the backward of workload 2's second half -- the input, weight and gamma gradients
# of the RMSNorm -> gate/up GEMM -> SwiGLU block -- with the block input h and the
# upstream gradient dy drawn directly (no first GEMM); 9: the backward of workload 2's
# whole chain (same forward draws as workload 2, then dy and the residual-stream
# gradient dres); 10: the backward of workload 6's second half -- the RMSNorm -> QKV
# GEMM -> RoPE block -- with h, W and dy drawn directly, positions as in workload 6;
# 11: the backward of workload 7's second half -- the RMSNorm -> LM head ->
# cross-entropy block -- with h, W and the targets drawn directly and the mean loss
# (row weights 1/M).
WORKLOADS = {
    1: Workload("tiny_m128_d256_n512_none", 128, 256, 256, 512, ACT_NONE, "bf16", 1e-5, 1001),
    2: Workload("llama1b_attnout_mlpin_m16384", 16384, 2048, 2048, 16384, ACT_SWIGLU, "bf16", 1e-5, 1002),
    3: Workload("llama1b_mlpout_qkv_m16384", 16384, 8192, 2048, 3072, ACT_NONE, "bf16", 1e-5, 1003),
    4: Workload("llama8b_attnout_mlpin_m16384", 16384, 4096, 4096, 28672, ACT_SWIGLU, "bf16", 1e-5, 1004),
    5: Workload("llama1b_attnout_mlpin_m16384_fp8", 16384, 2048, 2048, 16384, ACT_SWIGLU, "e4m3", 1e-5, 1002),
    6: Workload("llama1b_mlpout_qkv_rope_m16384", 16384, 8192, 2048, 3072, ACT_ROPE, "bf16", 1e-5, 1003,
                rot_cols=2560, seq_len=4096),
    7: Workload("llama1b_mlpout_lmhead_ce_m16384", 16384, 8192, 2048, 128256, ACT_CE, "bf16", 1e-5, 1007),
    8: Workload("llama1b_mlpin_bwd_m16384", 16384, 0, 2048, 16384, ACT_SWIGLU_BWD, "bf16", 1e-5, 1008),
    9: Workload("llama1b_attnout_mlpin_bwd_m16384", 16384, 2048, 2048, 16384, ACT_CHAIN_BWD, "bf16", 1e-5, 1002),
    10: Workload("llama1b_qkv_rope_bwd_m16384", 16384, 0, 2048, 3072, ACT_ROPE_BWD, "bf16", 1e-5, 1010,
                 rot_cols=2560, seq_len=4096),
    11: Workload("llama1b_lmhead_ce_bwd_m16384", 16384, 0, 2048, 128256, ACT_CE_BWD, "bf16", 1e-5, 1011),
}


def custom(M: int, K1: int, d: int, N2w: int, act: int, seed: int, dtype: str = "bf16",
           eps: float = 1e-5, rot_cols: int = 0, seq_len: int = 0) -> Workload:
    """A workload of arbitrary shape (ragged and edge-case tests)."""
    if act in (ACT_SWIGLU, ACT_SWIGLU_BWD, ACT_CHAIN_BWD) and N2w % 2:
        raise ValueError("SwiGLU needs an even number of second-weight rows")
    if act in (ACT_ROPE, ACT_ROPE_BWD) and (rot_cols % 64 or rot_cols > N2w or seq_len < 1):
        raise ValueError("RoPE needs whole 64-value heads within the columns and a sequence length")
    return Workload(f"custom_m{M}_k{K1}_d{d}_n{N2w}_a{act}", M, K1, d, N2w, act, dtype, eps, seed,
                    rot_cols=rot_cols, seq_len=seq_len)


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 array -> bf16 bit patterns (uint16), round-to-nearest-even via torch."""
    import torch

    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> fp32 values (exact widening)."""
    return (b.astype(np.uint32) << 16).view(np.float32)


def generate(w: Workload, rows: int | None = None) -> dict:
    """Draw the inputs of workload ``w``.

    Returns a dict of numpy arrays:
      A      uint16 [M, K1]   bf16 bits
      Wo_t   uint16 [d, K1]   bf16 bits (first weight, nn.Linear layout)
      x_res  uint16 [M, d]    bf16 bits
      gamma  float32 [d]
      W_t    uint16 [N2w, d]  bf16 bits (second weight before the gamma fold)
      pos    int32 [M]        RoPE workloads only: token m's position, m mod seq_len
      targets int32 [M]       cross-entropy workloads only: uniform in [0, N2w), drawn
                              after W
      dy     uint16 [M, N2w/2] whole-chain backward only: bf16 bits, N(0, 1), the
                              upstream gradient of y, drawn after W
      dres   uint16 [M, d]    whole-chain backward only: bf16 bits, N(0, 1), the gradient
                              reaching h through the residual stream, drawn after dy
    For an e4m3 workload these are the pre-quantisation tensors (quantisation is a
    step of the chain's weight/activation preparation, not of input generation).
    ``rows`` (optional) truncates M, keeping the draws of the first rows identical.
    """
    rng = np.random.default_rng(w.seed)
    f32 = np.float32
    if w.act in (ACT_SWIGLU_BWD, ACT_ROPE_BWD, ACT_CE_BWD):
        return _generate_bwd(w, rng, rows)
    A = rng.standard_normal((w.M, w.K1), dtype=f32)
    Wo = rng.standard_normal((w.d, w.K1), dtype=f32) * f32(1.0 / np.sqrt(w.K1))
    x = rng.standard_normal((w.M, w.d), dtype=f32)
    gamma = (f32(1.0) + f32(0.1) * rng.standard_normal(w.d, dtype=f32)).astype(f32)
    W = rng.standard_normal((w.N2w, w.d), dtype=f32) * f32(1.0 / np.sqrt(w.d))
    tgt = rng.integers(0, w.N2w, size=w.M, dtype=np.int32) if w.act == ACT_CE else None
    dy = dres = None
    if w.act == ACT_CHAIN_BWD:
        dy = rng.standard_normal((w.M, w.N2w // 2), dtype=f32)
        dres = rng.standard_normal((w.M, w.d), dtype=f32)
    if rows is not None:
        A, x = A[:rows], x[:rows]
        tgt = None if tgt is None else tgt[:rows]
        dy = None if dy is None else dy[:rows]
        dres = None if dres is None else dres[:rows]
    out = {
        "A": to_bf16_bits(A),
        "Wo_t": to_bf16_bits(Wo),
        "x_res": to_bf16_bits(x),
        "gamma": gamma,
        "W_t": to_bf16_bits(W),
    }
    if w.act == ACT_ROPE:
        out["pos"] = (np.arange(A.shape[0]) % w.seq_len).astype(np.int32)
    if tgt is not None:
        out["targets"] = tgt
    if dy is not None:
        out["dy"] = to_bf16_bits(dy)
        out["dres"] = to_bf16_bits(dres)
    return out


def _generate_bwd(w: Workload, rng, rows):
    """Inputs of the block-backward workloads, drawn in the order h, gamma, W, dy:
      h      uint16 [M, d]      bf16 bits, N(0, 1): the block's input (residual stream)
      gamma  float32 [d]        1 + 0.1 N(0, 1)
      W_t    uint16 [N2w, d]    bf16 bits, N(0, 1/d) (SwiGLU: gate rows, then up rows)
      dy     uint16 [M, n]      bf16 bits, N(0, 1): the upstream gradient of y (n = F for
                                SwiGLU, N2w for RoPE); cross-entropy: not drawn, instead
      targets int32 [M]         uniform in [0, N2w), and
      g      float32 [M]        1/M: the row weights of the mean loss
      pos    int32 [M]          RoPE only: token m's position, m mod seq_len
    """
    f32 = np.float32
    n = w.N2w // 2 if w.act == ACT_SWIGLU_BWD else w.N2w
    h = rng.standard_normal((w.M, w.d), dtype=f32)
    gamma = (f32(1.0) + f32(0.1) * rng.standard_normal(w.d, dtype=f32)).astype(f32)
    W = rng.standard_normal((w.N2w, w.d), dtype=f32) * f32(1.0 / np.sqrt(w.d))
    if w.act == ACT_CE_BWD:
        tgt = rng.integers(0, w.N2w, size=w.M, dtype=np.int32)
        if rows is not None:
            h, tgt = h[:rows], tgt[:rows]
        return {"h": to_bf16_bits(h), "gamma": gamma, "W_t": to_bf16_bits(W), "targets": tgt,
                "g": np.full(h.shape[0], 1.0 / w.M, dtype=f32)}
    dy = rng.standard_normal((w.M, n), dtype=f32)
    if rows is not None:
        h, dy = h[:rows], dy[:rows]
    out = {"h": to_bf16_bits(h), "gamma": gamma, "W_t": to_bf16_bits(W), "dy": to_bf16_bits(dy)}
    if w.act == ACT_ROPE_BWD:
        out["pos"] = (np.arange(h.shape[0]) % w.seq_len).astype(np.int32)
    return out
