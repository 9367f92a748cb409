"""Shared pieces of the GPU parity tests: build a paged case, run it, run the oracle.

Inputs come from ``workloads`` (seeded, generated on the device by torch), are
stored into the pool by ``kvd_write_kv`` and handed to the oracle in their
logical, contiguous form; nothing the oracle sees comes from the HIP path.
"""
from __future__ import annotations

import numpy as np
import torch

import decode_attention_paged_04_amd as kvd
import workloads as W
from oracle import attention, e4m3, numerics, paged, scores

DEV = "cuda"

# Tolerances.  Per element, the bf16 output is compared with the exact
# (float64, unrounded) oracle: |got - ref| <= max(4e-3, half a bf16 spacing at
# |ref| + the fp32 arithmetic's error).  Half a spacing is what rounding a
# correct fp32 result to bf16 may cost; where |ref| >= 1 it exceeds 4e-3 on its
# own, so no bf16 result could meet 4e-3 there.  Per output tensor of one
# layer call: relative L2 1e-3 against the oracle rounded to bf16 (nearest
# even) -- rounding exact values to bf16 alone gives a relative L2 of about
# 1.7e-3, so the 1e-3 bound can only hold against the rounded oracle.  FP8
# pools: relative L2 1e-2 against the oracle run on the same E4M3 codes (same
# per-element bound).  Cumulative scores: 1e-5 relative per element.
# The fp32 arithmetic's error is taken as TIE_REL * |ref| + TIE_ABS *
# max|ref| (2^-16 relative plus 2^-20 of the tensor's largest magnitude).
# Rounding ties: an exact value that lies within that error of a bf16
# rounding midpoint has two correct bf16 results.  A kernel value equal to the
# rounding of the reference moved by at most that error counts as exact in the
# relative L2.  In a small output tensor a single such flip of a large element
# would otherwise weigh more than 1e-3 on its own.
TIE_REL = 2.0 ** -16
TIE_ABS = 2.0 ** -20
TOL_MAX_ABS = 4e-3
TOL_REL_L2 = 1e-3
TOL_FP8_REL_L2 = 1e-2
TOL_SCORE_REL = 1e-5
TOL_LSE = 1e-5


def say(msg: str):
    print(msg, flush=True)


def bf16_to_f64(t) -> np.ndarray:
    return numerics.bf16_bits_to_f64(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def bf16_errors(got, ref_f64: np.ndarray):
    """(max-abs against the exact oracle, rel-L2 against the oracle rounded to
    bf16, worst element error over its allowance) of bf16 ``got`` (rounding
    ties, see TIE_REL, count as exact in the rel-L2)."""
    g = bf16_to_f64(got)
    ref = np.asarray(ref_f64, dtype=np.float64)
    r = numerics.round_to_bf16(ref)
    big = float(np.max(np.abs(ref))) if ref.size else 0.0
    t = TIE_REL * np.abs(ref) + TIE_ABS * big
    tie = (g == numerics.round_to_bf16(ref - t)) | (g == numerics.round_to_bf16(ref + t))
    denom = np.linalg.norm(r)
    e2 = np.where(tie, 0.0, np.abs(g - r))
    rel = float(np.linalg.norm(e2) / denom) if denom > 0 else float(np.linalg.norm(e2))
    if not g.size:
        return 0.0, rel, 0.0
    err = np.abs(g - ref)
    allow = np.maximum(TOL_MAX_ABS, 0.5 * numerics.bf16_ulp(ref) + t)
    return float(np.max(err)), rel, float(np.max(err / allow))


def assert_bf16_close(got, ref_f64, rel_tol=TOL_REL_L2, what=""):
    mx, rel, over = bf16_errors(got, ref_f64)
    assert over <= 1.0 and rel <= rel_tol, f"{what}: max-abs {mx:.3g} ({over:.2f} of allowance), rel-L2 {rel:.3g}"
    return mx, rel


def assert_lse_close(got, ref):
    g = got.detach().cpu().double().numpy()
    both_inf = np.isneginf(g) & np.isneginf(ref)
    fin = ~both_inf
    assert np.all(np.isfinite(g[fin])) and np.all(np.isfinite(ref[fin]))
    if fin.any():
        err = np.abs(g[fin] - ref[fin]) / np.maximum(1.0, np.abs(ref[fin]))
        assert float(np.max(err)) <= TOL_LSE, f"lse error {np.max(err):.3g}"


class PagedCase:
    """A seeded batch stored in a paged pool, plus what the oracle needs."""

    def __init__(self, w: W.DecodeWorkload, layers: int = None, lens=None, table=None,
                 num_blocks: int = None, poison: bool = True, keep_layers=None, keep_seqs=None):
        self.lens = np.asarray(lens if lens is not None else W.context_lengths(w), dtype=np.int32)
        if len(self.lens) != w.b:
            w = w.with_(b=len(self.lens))     # the batch is the given lengths
        self.w = w
        self.L = layers if layers is not None else w.layers
        if table is None:
            table, nb = W.block_tables(w, self.lens)
        else:
            nb = num_blocks
        self.table = np.asarray(table, dtype=np.int32)
        self.num_blocks = int(nb)
        self.fp8 = w.kv_dtype == "fp8"
        dt = kvd.KVD_FP8_E4M3 if self.fp8 else kvd.KVD_BF16
        self.pool = kvd.allocate_pool(self.L, self.num_blocks, w.n_kv, w.head_dim, dt)
        if poison:
            self.pool.kv.fill_(0xFF)          # NaN in every bf16 / E4M3 slot never written
        self.lens_t = torch.from_numpy(self.lens).to(DEV)
        self.table_t = torch.from_numpy(self.table).to(DEV)
        self.max_ctx = int(self.lens.max()) if len(self.lens) else 0
        self.offs = W.offsets(self.lens)
        slots = kvd.kvd_slot_mapping(self.table_t, self.lens_t)
        keep = set(range(self.L)) if keep_layers is None else set(keep_layers)
        self.keep_seqs = None if keep_seqs is None else sorted(set(int(i) for i in keep_seqs))
        self.q, self.kv, self.kv_seq = {}, {}, {}
        n = int(self.offs[-1])
        for layer in range(self.L):
            q = W.query(w, layer, DEV)
            K, V = W.keys_values(w, layer, n, DEV)
            kvd.kvd_write_kv(self.pool, layer, K, V, slots)
            self.q[layer] = q
            if layer in keep:
                if self.keep_seqs is None:
                    self.kv[layer] = (K.cpu(), V.cpu())
                else:
                    for i in self.keep_seqs:
                        lo, hi = int(self.offs[i]), int(self.offs[i + 1])
                        self.kv_seq[(layer, i)] = (K[lo:hi].cpu(), V[lo:hi].cpu())
            del K, V
        torch.cuda.synchronize()

    # ---------------------------------------------------------------- GPU
    def run(self, layer: int, chunk: int = 0, score=None, weight: float = 0.0, lse: bool = True):
        q = self.q[layer]
        out = torch.empty_like(q)
        lse_out = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV) if lse else None
        kvd.decode(self.pool, layer, q, self.table_t, self.lens_t, self.max_ctx, out=out,
                   lse_out=lse_out, chunk_tokens=chunk, score=score, score_weight=weight)
        return out, lse_out

    # ---------------------------------------------------------------- oracle
    def logical(self, layer: int, i: int):
        """float64 K, V ``[s][n_kv][d]`` of sequence i as the oracle sees them."""
        if (layer, i) in self.kv_seq:
            Ks, Vs = self.kv_seq[(layer, i)]
        else:
            K, V = self.kv[layer]
            lo, hi = int(self.offs[i]), int(self.offs[i + 1])
            Ks, Vs = K[lo:hi], V[lo:hi]
        Kf = bf16_to_f64(Ks)
        Vf = bf16_to_f64(Vs)
        if self.fp8:
            ck, sk = e4m3.quantize_sequence(Kf.astype(np.float32))
            cv, sv = e4m3.quantize_sequence(Vf.astype(np.float32))
            return e4m3.dequantize_sequence(ck, sk), e4m3.dequantize_sequence(cv, sv)
        return Kf, Vf

    def oracle(self, layer: int, seqs=None):
        if seqs is None:
            seqs = range(len(self.lens)) if self.keep_seqs is None else self.keep_seqs
        qf = bf16_to_f64(self.q[layer])
        o = np.zeros(qf.shape)
        lse = np.full(qf.shape[:2], -np.inf)
        for i in seqs:
            K, V = self.logical(layer, i)
            o[i], lse[i] = attention.decode_sequence(qf[i], K, V)
        return o, lse

    def oracle_alpha(self, layer: int, i: int):
        K, _ = self.logical(layer, i)
        return attention.attention_weights_sequence(bf16_to_f64(self.q[layer])[i], K)

    def oracle_scores(self, init: np.ndarray, seqs, weight: float):
        ref = init.astype(np.float64).copy()
        for i in seqs:
            s = int(self.lens[i])
            for layer in range(self.L):
                if s:
                    ref[i, :s] += scores.layer_increment(self.oracle_alpha(layer, i), weight)
        return ref

    def layout(self):
        return paged.PoolLayout(self.L, self.num_blocks, self.w.n_kv, self.w.head_dim,
                                elem_bytes=1 if self.fp8 else 2)


def score_rel_error(got: np.ndarray, ref: np.ndarray) -> float:
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), 1e-30))) if got.size else 0.0
