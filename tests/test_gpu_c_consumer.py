"""The C ABI from plain C: a C99 program (tests/c_demo/decode_demo.c, built by
build()) allocates device memory with the HIP runtime, creates a pool, stores
K/V with kvd_write_kv and runs kvd_decode_attn / kvd_decode_attn_fp8 -- no
Python and no PyTorch in the process that touches the GPU.  Its output must
match the float64 oracle on the same seeded inputs, to the tolerances of the
other parity tests."""
import os
import subprocess

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

HERE = os.path.dirname(os.path.abspath(__file__))
EXE = os.path.join(HERE, "c_demo", "decode_demo")


def _bits(t):
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("fp8,chunk", [(False, 0), (False, 64), (True, 0), (True, 96)])
def test_c_program_decode_matches_oracle(tmp_path, fp8, chunk):
    import gpu_harness as H
    import workloads as W
    from oracle import attention, e4m3
    assert os.path.exists(EXE), "the C consumer is not built: run __graft_entry__.build()"
    lens = np.array([300, 0, 1, 17, 1000, 48, 129], dtype=np.int32)
    w = W.DecodeWorkload("c_demo", seed=91 + int(fp8), b=len(lens), layers=1, n_q=16, n_kv=4, head_dim=128,
                         ctx=("fixed", 0), kv_dtype="fp8" if fp8 else "bf16")
    table, nb = W.block_tables(w, lens, pad_value=-1)
    offs = W.offsets(lens)
    n = int(offs[-1])
    q = W.query(w, 0, "cpu")
    K, V = W.keys_values(w, 0, n, "cpu")
    slots = np.concatenate([table[i, np.arange(s) // 16] * 16 + np.arange(s) % 16
                            for i, s in enumerate(lens)]).astype(np.int32)
    header = np.array([1 if fp8 else 0, w.b, w.n_q, w.n_kv, w.head_dim, nb, table.shape[1], n, chunk],
                      dtype=np.int32)
    src = tmp_path / "in.bin"
    dst = tmp_path / "out.bin"
    with open(src, "wb") as f:
        for a in (header, _bits(q), _bits(K), _bits(V), slots, table, lens):
            f.write(np.ascontiguousarray(a).tobytes())
    H.say(f"c consumer fp8={fp8} chunk={chunk}")
    r = subprocess.run([EXE, str(src), str(dst)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    H.say(r.stdout.strip())
    raw = np.fromfile(dst, dtype=np.uint8)
    nq = w.b * w.n_q * w.head_dim
    out = raw[:2 * nq].view(np.uint16).reshape(w.b, w.n_q, w.head_dim)
    lse = raw[2 * nq:].view(np.float32).reshape(w.b, w.n_q)
    qf = H.bf16_to_f64(q)
    ref_o = np.zeros(qf.shape)
    ref_l = np.full(qf.shape[:2], -np.inf)
    for i, s in enumerate(lens):
        lo, hi = int(offs[i]), int(offs[i + 1])
        Kf, Vf = H.bf16_to_f64(K[lo:hi]), H.bf16_to_f64(V[lo:hi])
        if fp8:
            ck, sk = e4m3.quantize_sequence(Kf.astype(np.float32))
            cv, sv = e4m3.quantize_sequence(Vf.astype(np.float32))
            Kf, Vf = e4m3.dequantize_sequence(ck, sk), e4m3.dequantize_sequence(cv, sv)
        if s:
            ref_o[i], ref_l[i] = attention.decode_sequence(qf[i], Kf, Vf)
    import torch
    got = torch.from_numpy(out.view(np.int16).copy()).view(torch.bfloat16)
    H.assert_bf16_close(got, ref_o, what=f"C consumer fp8={fp8} chunk={chunk}")
    H.assert_lse_close(torch.from_numpy(lse.copy()), ref_l)
