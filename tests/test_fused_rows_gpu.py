"""GPU parity of the single-pass forward + backward (grpo_logits_fwd_bwd)
against the float64 oracle, with the tolerances of test_rows_gpu.py."""
import numpy as np
import pytest
import torch

import oracle
import synth
from gpu_common import GrpoInputs, dev, logits_to_dev, require_gpu, say
from test_rows_gpu import _tiny, _token_case, check_backward, check_forward, oracle_expectations

pytestmark = pytest.mark.gpu


def run_single_pass(lib, t, inp: GrpoInputs, force_dense=False, dlogits=None):
    c = inp.case
    d = inp.to_dev()
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    o, dz, zr = lib.grpo_logits_fwd_bwd(t, d["ids"], d["old_logp"], d["adv"], c.B, c.L, d["dloss"],
                                        ref_logp=d["ref_logp"], mask=d["mask"],
                                        temperature=c.temperature, beta=c.beta,
                                        eps_low=c.eps_low, eps_high=c.eps_high,
                                        force_dense=force_dense, dlogits=dlogits, err_count=err)
    torch.cuda.synchronize()
    o["err_count"] = err
    return o, dz, zr


@pytest.mark.parametrize("variant", ["a", "b", "c", "t"])
def test_single_pass_tiny(variant):
    lib = require_gpu()
    case, z64, inp = _tiny(variant)
    say(f"single-pass tiny: variant {variant}")
    o, dz, zr = run_single_pass(lib, logits_to_dev(case.logits, "f32"), inp)
    ox, g = oracle_expectations(inp, z64, o)
    check_forward(case, ox, o, ref=inp.ref)
    check_backward(case, ox, g, dz, zr, z64, inp)


def test_single_pass_rejects_sequence_level():
    lib = require_gpu()
    case, z64, inp = _tiny("s")
    d = inp.to_dev()
    t = logits_to_dev(case.logits, "f32")
    import ctypes
    from rl_fine_tuning_row_amd._lib import GrpoParams, _ptr
    p = GrpoParams(1.0, 0.04, 0.2, 0.2, 1, 0)
    buf = torch.empty(case.N, device="cuda")
    st = lib.lib().grpo_logits_fwd_bwd(_ptr(t), 0, case.B, case.L, case.V, case.V, _ptr(d["ids"]),
                                       _ptr(d["old_logp"]), None, _ptr(d["adv"]), None,
                                       ctypes.byref(p), _ptr(d["dloss"]), _ptr(buf), _ptr(buf),
                                       _ptr(buf), None, None, None, _ptr(torch.empty_like(t)),
                                       case.V, None, None, None)
    assert st == 8  # GRPO_ERR_PARAM


@pytest.mark.parametrize("with_ref", [False, True])
@pytest.mark.parametrize("dloss", ["sum", "mean"])
def test_single_pass_token_level(with_ref, dloss):
    lib = require_gpu()
    case, inp = _token_case(with_ref, dloss)
    say(f"single-pass B4 L512 V32000 bf16, ref={'noise' if with_ref else 'policy'}, dloss={dloss}")
    t = logits_to_dev(case.logits, "bf16")
    o, dz, zr = run_single_pass(lib, t, inp)
    z64 = oracle.decode_bf16(case.logits)
    ox, g = oracle_expectations(inp, z64, o)
    check_forward(case, ox, o, ref=inp.ref)
    check_backward(case, ox, g, dz, zr, z64, inp)
    # early path vs forced dense: torch.equal
    _, dz2, zr2 = run_single_pass(lib, t, inp, force_dense=True)
    assert torch.equal(dz, dz2) and torch.equal(zr, zr2)
    # in place
    tt = t.clone()
    run_single_pass(lib, tt, inp, dlogits=tt)
    assert torch.equal(tt.view(torch.int16), dz.view(torch.int16))


@pytest.mark.parametrize("dtype,V,ld_extra", [("bf16", 70008, 0), ("f32", 40000, 0),
                                             ("bf16", 65536, 0), ("bf16", 65544, 0),
                                             ("f32", 32768, 0), ("f32", 32772, 0),
                                             ("bf16", 40003, 5), ("bf16", 20011, 5),
                                             ("f32", 12003, 5),
                                             ("bf16", 1003, 0), ("f32", 17, 0),
                                             ("bf16", 1003, 1)])
def test_single_pass_shapes(dtype, V, ld_extra):
    """Rows too long for registers or not 16-byte aligned take the two-pass
    path inside the same call; ragged tails on 16-byte aligned rows (input and
    output pitch V + ld_extra) take the single pass: 5000 vectors at 512 x 16,
    2501 at 1024 x 4.  65536 bf16 / 32768 fp32 (8192 vectors) is the longest
    row held in registers; one vector more takes the two-pass path."""
    lib = require_gpu()
    say(f"single-pass shapes: {dtype} V={V} ld=V+{ld_extra}")
    _edge_case(lib, dtype, V, ld_extra, 0.9, out_pitch=ld_extra > 0 and V > 2000)


@pytest.mark.parametrize("dtype,V", [("bf16", 16003), ("f32", 8003)])
@pytest.mark.parametrize("shape", ["256,8", "256,16", "512,8", "512,16", "1024,4"])
def test_single_pass_every_shape(shape, dtype, V, monkeypatch):
    """Every compiled (workgroup, vectors per lane) shape of the single pass,
    forced through the library's launch override, on a row of 2000 vectors
    plus a 3-element tail that fits all of them (16-byte pitch V + 5)."""
    lib = require_gpu()
    monkeypatch.setenv("GRPO_ROWS_FUSED_LAUNCH", shape)
    say(f"single-pass shape {shape}: {dtype} V={V} ld={V + 5}")
    _edge_case(lib, dtype, V, 5, 0.9, out_pitch=True)


@pytest.mark.parametrize("dtype,V,pad", [("bf16", 2048, 0), ("bf16", 2047, 1), ("f32", 1024, 0),
                                         ("f32", 1027, 1), ("bf16", 2056, 0), ("f32", 1028, 0)])
def test_single_pass_one_wave(dtype, V, pad):
    """Rows of up to 256 vectors take one 64-lane wave with 4 vectors per
    lane (no cross-wave merge): exactly 256 vectors, 255 plus a 7-element
    tail and 256 plus a 3-element tail (16-byte pitch V + pad for input and
    output); 257 vectors take 256 lanes x 8."""
    lib = require_gpu()
    say(f"single-pass one wave: {dtype} V={V} ld=V+{pad}")
    _edge_case(lib, dtype, V, pad, 0.9, out_pitch=pad > 0)


@pytest.mark.parametrize("dtype,V", [("bf16", 40), ("bf16", 1003), ("f32", 17), ("f32", 200)])
@pytest.mark.parametrize("T", [0.05, 0.1, 0.3, 0.5, 0.7, 1.0, 1.3, 2.0, 10.0])
def test_single_pass_lanes_without_elements(dtype, V, T):
    """Rows shorter than the workgroup leave lanes with no element.  Such a lane
    once folded its fill values into garbage sums (the rounding error of
    fill * log2e / T, positive for some temperatures -> inf -> NaN after the
    merge); it must contribute nothing at every temperature.  Every other row
    samples its most likely token, so at the low temperatures logp is close
    to 0 and its 1e-6 floor binds (a lane's sums referenced to the rounded
    fl(m log2e / T) instead of the exact max missed it by up to 5e-6)."""
    lib = require_gpu()
    say(f"single-pass short rows: {dtype} V={V} T={T}")
    _edge_case(lib, dtype, V, 0, T, argmax=True)


@pytest.mark.parametrize("dtype,V,ld_extra", [("bf16", 32000, 0), ("bf16", 16003, 5),
                                             ("f32", 8003, 5), ("f32", 4096, 0)])
@pytest.mark.parametrize("T", [0.05, 0.1])
def test_single_pass_low_temperature(dtype, V, ld_extra, T):
    """Rows of thousands of vectors at T = 0.05 and 0.1 with every other row
    sampling its most likely token (logp close to 0)."""
    lib = require_gpu()
    say(f"single-pass low temperature: {dtype} V={V} ld=V+{ld_extra} T={T}")
    _edge_case(lib, dtype, V, ld_extra, T, out_pitch=ld_extra > 0, argmax=True)


def _edge_case(lib, dtype, V, ld_extra, T, out_pitch=False, argmax=False):
    B, L = 2, 3
    rng = np.random.default_rng(V)
    zf = (rng.standard_normal((B * L, V + ld_extra)) * 2.0).astype(np.float32)
    zb = synth.f32_to_bf16_bits(zf) if dtype == "bf16" else zf
    t = logits_to_dev(zb, dtype)[:, :V]
    z64 = oracle.to_f64(zb, dtype)[:, :V]
    ids = rng.integers(0, V, B * L).astype(np.int64)
    if argmax:
        ids[::2] = z64[::2].argmax(axis=1)
    lp, _ = oracle.selective_log_softmax(z64, ids, T)
    case = synth.GrpoCase(name="edge", B=B, L=L, V=V, dtype=dtype, logits=None, ids=ids,
                          adv=np.array([0.7, -1.1], np.float32), mask=np.ones(B * L, np.uint8),
                          old_noise=rng.standard_normal(B * L) * 0.2,
                          ref_noise=rng.standard_normal(B * L) * 0.1,
                          dloss=np.ones(B * L, np.float32), temperature=T, beta=0.04,
                          eps_low=0.2, eps_high=0.28, level="token")
    inp = GrpoInputs(case, lp)
    dl = None
    if out_pitch:  # dlogits with the same padded pitch as the logits
        dl = torch.empty((B * L, V + ld_extra), dtype=t.dtype, device="cuda")[:, :V]
    o, dz, zr = run_single_pass(lib, t, inp, dlogits=dl)
    ox, g = oracle_expectations(inp, z64, o)
    check_forward(case, ox, o, ref=inp.ref)
    check_backward(case, ox, g, dz, zr, z64, inp)
