"""Seeded synthetic inputs for the selective scans.

This module is the one thing the oracle side and the GPU side share. It holds
none of the method's arithmetic: only random draws, dtype rounding (bf16 by
round-to-nearest-even through torch on the CPU) and shape bookkeeping.

Every tensor of every sequence has its own numpy generator,
``default_rng(SeedSequence([workload_key, tensor_id, sequence]))``, so any subset
of sequences regenerates on its own (the oracle checks samples of the large
workloads that way).

Distributions (the same for every workload unless a workload says otherwise):

* x ~ N(0, 1)                         hidden states / scan input [tokens, D]
* dt_raw ~ N(-2, 0.5)                 raw step input [tokens, D]; Delta = softplus(dt_raw)
                                      is applied by the scan itself
* A[d, n] = -(n + 1)                  S4D-real initialisation [D, N]
* Bm, Cm ~ N(0, 1)                    [tokens, N], shared by all channels
* Dskip ~ N(0, 1)                     [D]
"""
from __future__ import annotations

import dataclasses

import numpy as np

# tensor ids inside a workload's seed tree
X, DT, BM, CM, DSKIP, RES, GATE, LENS, HIN, PLENS = range(10)


def rng(key: int, tensor_id: int, seq: int = 0) -> np.random.Generator:
    return np.random.default_rng(np.random.SeedSequence([int(key), int(tensor_id), int(seq)]))


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 array -> fp32 array holding the bf16 round-to-nearest-even values."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def as_dtype(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    return round_bf16(a) if dtype == "bf16" else a


def offsets(lengths) -> np.ndarray:
    lengths = np.asarray(lengths, dtype=np.int64)
    off = np.zeros(lengths.shape[0] + 1, dtype=np.int64)
    np.cumsum(lengths, out=off[1:])
    return off


def s4d_real_A(D: int, N: int) -> np.ndarray:
    """A[d, n] = -(n + 1) for every channel."""
    return np.tile(-(np.arange(N, dtype=np.float32) + 1.0), (D, 1))


@dataclasses.dataclass
class ScanInputs:
    """One batch of scan inputs. Float arrays are fp32 numpy arrays that hold
    exactly the values the kernel sees (already bf16-rounded for bf16)."""
    dtype: str
    lengths: np.ndarray          # [batch] int64
    offsets: np.ndarray          # [batch+1] int64
    x: np.ndarray                # [tokens, D]
    dt: np.ndarray               # [tokens, D] raw (pre-softplus)
    Bm: np.ndarray               # [tokens, N]
    Cm: np.ndarray               # [tokens, N]
    A: np.ndarray                # [D, N] fp32
    Dskip: np.ndarray            # [D] fp32

    @property
    def batch(self) -> int:
        return int(self.lengths.shape[0])

    @property
    def tokens(self) -> int:
        return int(self.offsets[-1])

    @property
    def D(self) -> int:
        return int(self.A.shape[0])

    @property
    def N(self) -> int:
        return int(self.A.shape[1])

    def rows(self, b: int) -> slice:
        return slice(int(self.offsets[b]), int(self.offsets[b + 1]))

    def subset(self, seqs) -> "ScanInputs":
        """The listed sequences only (re-packed), for sampled oracle checks."""
        seqs = list(seqs)
        idx = np.concatenate([np.arange(self.offsets[b], self.offsets[b + 1]) for b in seqs]) \
            if seqs else np.zeros(0, dtype=np.int64)
        lens = self.lengths[seqs]
        return ScanInputs(self.dtype, lens, offsets(lens), self.x[idx], self.dt[idx],
                          self.Bm[idx], self.Cm[idx], self.A, self.Dskip)


def scan_inputs(key: int, lengths, D: int, N: int = 16, dtype: str = "f32",
                dt_mean: float = -2.0, dt_std: float = 0.5, seqs=None) -> ScanInputs:
    """Draw x, dt, Bm, Cm per sequence and A, Dskip per workload.

    ``seqs``: generate only these sequence indices (their draws are identical
    to the ones in the full batch).
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    if seqs is None:
        seqs = range(lengths.shape[0])
    seqs = list(seqs)
    xs, dts, bs, cs = [], [], [], []
    for b in seqs:
        L = int(lengths[b])
        xs.append(rng(key, X, b).standard_normal((L, D), dtype=np.float32))
        dts.append((rng(key, DT, b).standard_normal((L, D), dtype=np.float32) * dt_std + dt_mean)
                   .astype(np.float32))
        bs.append(rng(key, BM, b).standard_normal((L, N), dtype=np.float32))
        cs.append(rng(key, CM, b).standard_normal((L, N), dtype=np.float32))
    cat = (lambda parts, w: np.concatenate(parts, axis=0) if parts
           else np.zeros((0, w), dtype=np.float32))
    lens = lengths[seqs]
    return ScanInputs(
        dtype=dtype, lengths=lens, offsets=offsets(lens),
        x=as_dtype(cat(xs, D), dtype), dt=as_dtype(cat(dts, D), dtype),
        Bm=as_dtype(cat(bs, N), dtype), Cm=as_dtype(cat(cs, N), dtype),
        A=s4d_real_A(D, N),
        Dskip=rng(key, DSKIP).standard_normal(D, dtype=np.float32))


def uniform_lengths(key: int, tensor_id: int, batch: int, lo: int, hi: int) -> np.ndarray:
    """batch integer lengths drawn uniformly from [lo, hi] inclusive."""
    return rng(key, tensor_id).integers(lo, hi + 1, size=batch).astype(np.int64)


def gates(key: int, count: int, lo: float, hi: float) -> np.ndarray:
    """Residual gates s ~ U(lo, hi), one per hook, as fp32."""
    return rng(key, GATE).uniform(lo, hi, size=count).astype(np.float32)


def initial_state(key: int, batch: int, D: int, N: int, scale: float = 1.0) -> np.ndarray:
    """A cached boundary state stand-in, N(0, scale^2), fp32 [batch, D, N]."""
    return (rng(key, HIN).standard_normal((batch, D, N), dtype=np.float32) * scale).astype(np.float32)


# --------------------------------------------------------------------------
# The workloads. Each is named for what it is and carries its sizes.
# --------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Workload:
    key: int
    name: str
    desc: str


TINY = Workload(100, "tiny_r2l_fp32_b1_L64_D64_N16",
                "full-sequence reverse scan, fp32, batch 1, L=64, D=64, N=16, res=x, s=0.5")
BLOCK = Workload(101, "block_restricted_fp32_b8_P512_T32_D256_N16",
                 "fp32, batch 8: forward prefix scan over 512 tokens to a boundary state "
                 "[256, 16], then a reverse scan over one active block of 32 tokens")
DENOISE = Workload(102, "denoise_step_bf16_b64_blk32_D2048_N16_7hooks",
                   "R2LM denoising step: batch 64, generation block 32, D=2048, N=16, bf16 "
                   "inputs, fp32 state; 7 hooked reverse scans (every 4th of 28 layers), "
                   "res = x, s ~ U(0, 0.1) per hook")
PREFILL = Workload(103, "prefill_r2l_bf16_b8_L4096_D4096_N16",
                   "full reverse scan, batch 8, L=4096, D=4096, N=16, bf16, fp32 state, out = y")
RAGGED = Workload(104, "ragged_serving_bf16_b256_blk16to64_D4096_N16",
                  "batch 256, active blocks of U{16..64} tokens, D=4096, N=16, bf16: reverse "
                  "scan over the blocks (out = y) and block_commit_state over each block; "
                  "prefixes of U{256..8192} tokens for the prefill that builds the states")

BIDIR = Workload(105, "bidir_window_step_bf16_b64_L32_D2048_N16_7hooks",
                 "bidirectional full-window scans over the denoising window: batch 64, 32 "
                 "tokens, D=2048, N=16, bf16 inputs, fp32 state, 7 hooked layers; the forward "
                 "and the reverse direction each with its own dt, Bm, Cm, A, Dskip; res = x, "
                 "s ~ U(0, 0.1) per hook")

SIDECAR = Workload(106, "sidecar_step_bf16_b64_blk32_dm2048_di4096_N16_7hooks",
                   "R2LM denoising step with the whole sidecar block per hook: batch 64, "
                   "generation block 32, d_model 2048 (the hook's hidden width), d_inner 4096, "
                   "N=16, dt_rank 128, conv width 4, bf16 activations and projection weights, "
                   "fp32 state; 7 hooks, out = hidden + s * block(hidden), s ~ U(0, 0.1)")

WORKLOADS = {w.name: w for w in (TINY, BLOCK, DENOISE, PREFILL, RAGGED, BIDIR, SIDECAR)}


def tiny_inputs() -> ScanInputs:
    return scan_inputs(TINY.key, [64], D=64, N=16, dtype="f32")


def block_inputs():
    """(prefix inputs [8 x 512], block inputs [8 x 32]) of the block-restricted workload."""
    pre = scan_inputs(BLOCK.key, [512] * 8, D=256, N=16, dtype="f32")
    blk = scan_inputs(BLOCK.key + 1000, [32] * 8, D=256, N=16, dtype="f32")
    return pre, blk


def denoise_hook_inputs(hook: int, seqs=None) -> ScanInputs:
    return scan_inputs(DENOISE.key * 100 + hook, [32] * 64, D=2048, N=16, dtype="bf16", seqs=seqs)


def denoise_gates() -> np.ndarray:
    return gates(DENOISE.key, 7, 0.0, 0.1)


def prefill_inputs(seqs=None) -> ScanInputs:
    return scan_inputs(PREFILL.key, [4096] * 8, D=4096, N=16, dtype="bf16", seqs=seqs)


def ragged_block_lengths() -> np.ndarray:
    return uniform_lengths(RAGGED.key, LENS, 256, 16, 64)


def ragged_prefix_lengths() -> np.ndarray:
    return uniform_lengths(RAGGED.key, PLENS, 256, 256, 8192)


def ragged_block_inputs(seqs=None) -> ScanInputs:
    return scan_inputs(RAGGED.key, ragged_block_lengths(), D=4096, N=16, dtype="bf16", seqs=seqs)


def ragged_commit_inputs(seqs=None) -> ScanInputs:
    """The committed (now clean) blocks: same lengths, independent draws."""
    return scan_inputs(RAGGED.key + 1000, ragged_block_lengths(), D=4096, N=16, dtype="bf16",
                       seqs=seqs)


def ragged_prefix_inputs(seqs=None) -> ScanInputs:
    return scan_inputs(RAGGED.key + 2000, ragged_prefix_lengths(), D=4096, N=16, dtype="bf16",
                       seqs=seqs)


def reverse_params(key: int, lengths, D: int, N: int = 16, dtype: str = "f32",
                   dt_mean: float = -2.0, seqs=None) -> dict:
    """The reverse direction's own parameters for a bidirectional scan over
    inputs drawn with ``key``: dt, Bm, Cm and Dskip drawn independently, A the
    S4D-real matrix at half the rates (so that the two directions differ)."""
    r = scan_inputs(key + 5000, lengths, D, N, dtype, dt_mean=dt_mean, seqs=seqs)
    return {"dt": r.dt, "Bm": r.Bm, "Cm": r.Cm, "A": (0.5 * r.A).astype(np.float32),
            "Dskip": r.Dskip}


def bidir_inputs(hook: int = 0, seqs=None) -> ScanInputs:
    return scan_inputs(BIDIR.key * 100 + hook, [32] * 64, D=2048, N=16, dtype="bf16", seqs=seqs)


def bidir_reverse(hook: int = 0, seqs=None) -> dict:
    return reverse_params(BIDIR.key * 100 + hook, [32] * 64, D=2048, N=16, dtype="bf16",
                          seqs=seqs)


def bidir_gates() -> np.ndarray:
    return gates(BIDIR.key, 7, 0.0, 0.1)


def sidecar_weights(key: int, dm: int, di: int, R: int, N: int = 16, K: int = 4,
                    dtype: str = "f32") -> dict:
    """Random-init weights of the sidecar block (no trained weights exist):
    projections N(0, 1/fan_in) stored [out, in] in ``dtype``; conv taps N(0, 1/K),
    conv bias N(0, 0.1^2), dt bias N(-2, 0.5^2) (Delta ~ softplus(-2) at
    init), A = S4D-real, Dskip N(0, 1), all fp32."""
    g = lambda t: rng(key, 50 + t)   # noqa: E731
    f32 = lambda a: np.asarray(a, dtype=np.float32)   # noqa: E731
    return {
        "W_in": as_dtype(f32(g(0).standard_normal((2 * di, dm)) / np.sqrt(dm)), dtype),
        "conv_w": f32(g(1).standard_normal((di, K)) / np.sqrt(K)),
        "conv_b": f32(g(2).standard_normal(di) * 0.1),
        "W_x": as_dtype(f32(g(3).standard_normal((R + 2 * N, di)) / np.sqrt(di)), dtype),
        "W_dt": as_dtype(f32(g(4).standard_normal((di, R)) / np.sqrt(R)), dtype),
        "dt_bias": f32(g(5).normal(-2.0, 0.5, di)),
        "A": s4d_real_A(di, N),
        "Dskip": f32(g(6).standard_normal(di)),
        "W_out": as_dtype(f32(g(7).standard_normal((dm, di)) / np.sqrt(di)), dtype),
    }


def hidden_states(key: int, lengths, dm: int, dtype: str = "f32") -> np.ndarray:
    """Stand-in hidden states [tokens, dm] ~ N(0, 1), one generator per sequence."""
    parts = [rng(key, X, b).standard_normal((int(L), dm), dtype=np.float32)
             for b, L in enumerate(lengths)]
    a = np.concatenate(parts, axis=0) if parts else np.zeros((0, dm), dtype=np.float32)
    return as_dtype(a, dtype)


def sidecar_hook(hook: int):
    """(hidden [2048, 2048] bf16 values, weights, s) of one hook of the sidecar step."""
    key = SIDECAR.key * 100 + hook
    return (hidden_states(key, [32] * 64, 2048, "bf16"),
            sidecar_weights(key, 2048, 4096, 128, dtype="bf16"),
            float(gates(SIDECAR.key, 7, 0.0, 0.1)[hook]))
