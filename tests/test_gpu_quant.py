"""GPU: the quantized attention form.

Encodings (int8 Q/K codes and block scales, E4M3 V codes and channel scales) are bit-exact
with the oracle's quantizers; the quantized forward meets the cosine gate (>= 0.999) against
the unquantized fp64 oracle, and tracks the oracle's dequantized-input attention closely.
"""
import numpy as np
import pytest

from oracle import attention as ref_attn
from oracle import quant as ref_q
from tests._util import cosine, to_device
from workloads import make_workload, random_case

pytestmark = pytest.mark.gpu


def _fa():
    import block_sparse_masked_blockmask_amd as fa
    return fa


def _quantize(w):
    import torch
    fa = _fa()
    dev = torch.device("cuda", 0)
    q, k, v = (to_device(x, "bf16", dev) for x in (w.q, w.k, w.v))
    out = fa.flexattn_quantize_qkv(q, k, v)
    torch.cuda.synchronize()
    return (q, k, v), {key: t.cpu().numpy() for key, t in out.items()}, out


@pytest.mark.parametrize("L", [333, 128, 700])
def test_encodings_bit_exact(L):
    w = random_case(800 + L, dtype="bf16", B=2, Hq=3, Hkv=3, Lq=L)
    qf, kf, vf = w.qkv_f32()
    vf = vf * np.linspace(0.01, 3.0, 128, dtype=np.float32)[None, None, None, :]
    from workloads import f32_to_bf16_bits
    w.v = f32_to_bf16_bits(vf)
    vf = w.qkv_f32()[2]
    qf = qf.copy()
    # An all-zero block (scale 0, codes 0) in Q.
    w.q = w.q.copy()
    w.q[1, 2, :min(128, L)] = 0
    qf[1, 2, :min(128, L)] = 0
    _, got, _ = _quantize(w)
    for name, x in (("q", qf), ("k", kf)):
        codes, scales = ref_q.quantize_int8_blocks(x)
        assert np.array_equal(got[name + "_scale"], scales), name
        assert np.array_equal(got[name + "8"], codes), name
    codes, scales = ref_q.quantize_fp8_channels(vf)
    assert np.array_equal(got["v_scale"], scales)
    assert np.array_equal(got["v8"], codes)


def _quant_fwd(dev_out, w, qkv):
    import torch
    fa = _fa()
    out, lse = fa.flexattn_fwd(dev_out["q8"], dev_out["k8"], dev_out["v8"], q_scale=dev_out["q_scale"],
                               k_scale=dev_out["k_scale"], v_scale=dev_out["v_scale"])
    torch.cuda.synchronize()
    return out.float().cpu().numpy(), lse.cpu().numpy()


@pytest.mark.parametrize("shape", [(1, 4, 4, 300, 300), (2, 8, 2, 257, 513)])
def test_quantized_forward_small(shape):
    B, Hq, Hkv, Lq, Lkv = shape
    w = random_case(900 + Lq, dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, Lq=Lq, Lkv=Lkv)
    qkv, got, dev_out = _quantize(w)
    out, lse = _quant_fwd(dev_out, w, qkv)
    qf, kf, vf = w.qkv_f32()
    o_ref, l_ref = ref_attn.attention(qf, kf, vf, {})
    c = cosine(out, o_ref)
    assert c >= 0.999, c
    assert np.abs(lse - l_ref).max() < 5e-2
    # Diagnostic (equal head counts): the oracle on the dequantized inputs, P rounded through E4M3.
    # The kernel rounds P relative to the running maximum of the online softmax, the oracle
    # relative to the final row maximum, so the two roundings of P differ by up to one E4M3
    # step (2^-4 relative); the bound reflects that, not the rounding-free 0.99999.
    if Hq == Hkv:
        for b, h in [(0, 0), (B - 1, Hq - 1)]:
            rows = np.arange(0, Lq, 7)
            o_dq = ref_q.attention_dequantized(got["q8"], got["q_scale"], got["k8"], got["k_scale"], got["v8"],
                                               got["v_scale"], rows, b, h, round_p=True)
            assert cosine(out[b, h, rows], o_dq) >= 0.9995


def test_quantized_forward_refusals():
    import torch
    fa = _fa()
    w = random_case(950, dtype="bf16", B=1, Hq=2, Lq=130)
    _, _, dev_out = _quantize(w)
    with pytest.raises(fa.FlexAttnError) as e:
        fa.flexattn_fwd(dev_out["q8"], dev_out["k8"], dev_out["v8"], None, fa.FA_MASK_CAUSAL,
                        q_scale=dev_out["q_scale"], k_scale=dev_out["k_scale"], v_scale=dev_out["v_scale"])
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    with pytest.raises(fa.FlexAttnError) as e:
        fa.flexattn_fwd(dev_out["q8"], dev_out["k8"], dev_out["v8"], None, 0, fa.FA_SCORE_SOFTCAP, softcap=5.0,
                        q_scale=dev_out["q_scale"], k_scale=dev_out["k_scale"], v_scale=dev_out["v_scale"])
    assert e.value.status == fa.FA_ERR_UNSUPPORTED
    with pytest.raises(fa.FlexAttnError) as e:
        fa.flexattn_fwd(dev_out["q8"], dev_out["k8"], dev_out["v8"])
    assert e.value.status == fa.FA_ERR_INVALID_ARG


def test_dense_workload_quantized_full_size():
    print("workload dense_b1h32s24576_bf16 (quantized)", flush=True)
    w = make_workload("dense_b1h32s24576_bf16")
    qkv, got, dev_out = _quantize(w)
    out, lse = _quant_fwd(dev_out, w, qkv)
    qf, kf, vf = w.qkv_f32()
    # Encodings bit-exact on sampled heads.
    for h in (0, 17, 31):
        codes, scales = ref_q.quantize_int8_blocks(qf[:, h:h + 1])
        assert np.array_equal(got["q8"][:, h:h + 1], codes) and np.array_equal(got["q_scale"][:, h:h + 1], scales)
        codes, scales = ref_q.quantize_fp8_channels(vf[:, h:h + 1])
        assert np.array_equal(got["v8"][:, h:h + 1], codes) and np.array_equal(got["v_scale"][:, h:h + 1], scales)
    rng = np.random.default_rng(5)
    gots, wants = [], []
    for h in rng.choice(32, 4, replace=False):
        rows = np.sort(rng.choice(w.Lq, 64, replace=False))
        o_ref, _ = ref_attn.attention_rows(qf, kf, vf, {}, 0, int(h), rows)
        gots.append(out[0, h, rows])
        wants.append(o_ref)
    c = cosine(np.concatenate(gots), np.concatenate(wants))
    print(f"quantized cosine vs unquantized oracle: {c:.6f}")
    assert c >= 0.999
