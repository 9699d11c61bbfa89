"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device."""
import os
import re

import pytest

from qwen3_kv_cache_amd import qdec

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "qdec.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(qdec_[a-z_]+)\s*\(", src)))


def test_header_declares_the_binding_exports():
    assert declared_functions() == sorted(qdec.EXPORTS)


def test_library_exports_every_declared_symbol():
    L = qdec.lib()
    for name in declared_functions():
        assert hasattr(L, name), name


def test_header_compiles_as_c():
    import shutil
    import subprocess
    import tempfile
    gcc = shutil.which("gcc")
    if not gcc:
        pytest.skip("gcc missing")
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "t.c")
        open(c, "w").write('#include "qdec.h"\nint main(void){qdec_config c; (void)c; return QDEC_OK;}\n')
        r = subprocess.run([gcc, "-std=c99", "-Wall", "-Werror", "-I", os.path.dirname(HEADER), c, "-o",
                            os.path.join(d, "t")], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr


def good_cfg(**kw):
    base = dict(hidden=128, n_layer=2, n_q_head=4, n_kv_head=2, head_dim=32, ffn=384, vocab=1024)
    base.update(kw)
    bf16 = base.pop("bf16", True)
    tied = base.pop("tied", 1)
    return qdec.make_config(bf16=bf16, tied=tied, **base)


BAD = [
    dict(tied=0), dict(hidden=100), dict(hidden=0), dict(head_dim=48), dict(head_dim=256), dict(n_kv_head=3),
    dict(n_q_head=32, n_kv_head=2), dict(ffn=100), dict(vocab=1), dict(n_layer=0),
    dict(rms_eps=0.0), dict(rope_theta=0.5),
    # limits of the decode kernel: hidden <= 1024, n_kv_head <= 8, GQA group <= 4, ffn % 64 == 0, ffn <= 8192
    dict(hidden=2048), dict(n_q_head=16, n_kv_head=16), dict(n_q_head=16, n_kv_head=2), dict(ffn=96), dict(ffn=8256),
]


@pytest.mark.parametrize("kw", BAD, ids=[str(k) for k in BAD])
def test_create_rejects_bad_config(kw):
    cfg = good_cfg(**kw)
    table = qdec.WeightTable(0, 0, [[0] * qdec.QDEC_W_PER_LAYER] * 2)
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_create(cfg, table.c, 0)
    assert e.value.code == qdec.QDEC_E_INVALID
    assert qdec.qdec_last_error()


def test_create_rejects_q8_with_ffn_not_whole_blocks():
    # Q8_0 weights: each of the down projection's 8 input slices must be whole
    # 32-input blocks, so ffn must be a multiple of 256 (384 is not)
    cfg = good_cfg(ffn=384)
    cfg.weight_dtype = qdec.QDEC_Q8_0
    table = qdec.WeightTable(0, 0, [[0] * qdec.QDEC_W_PER_LAYER] * 2)
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_create(cfg, table.c, 0)
    assert e.value.code == qdec.QDEC_E_INVALID and "Q8_0" in qdec.qdec_last_error()
    # with ffn 512 the config passes and the null weights are what is rejected
    cfg = good_cfg(ffn=512)
    cfg.weight_dtype = qdec.QDEC_Q8_0
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_create(cfg, table.c, 0)
    assert e.value.code == qdec.QDEC_E_INVALID and "weights" in qdec.qdec_last_error()


def test_create_rejects_bad_dtype_and_null_weights():
    cfg = good_cfg()
    cfg.weight_dtype = 7
    table = qdec.WeightTable(0, 0, [[0] * qdec.QDEC_W_PER_LAYER] * 2)
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_create(cfg, table.c, 0)
    assert e.value.code == qdec.QDEC_E_INVALID and "weight_dtype" in qdec.qdec_last_error()
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_create(good_cfg(), table.c, 0)
    assert e.value.code == qdec.QDEC_E_INVALID and "weights" in qdec.qdec_last_error()


def test_null_handles_are_rejected():
    L = qdec.lib()
    assert L.qdec_state_pos(None) == -1
    assert L.qdec_destroy(None) == qdec.QDEC_OK
    L.qdec_state_destroy(None)  # no-op
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_state_create(0, 16)
    assert e.value.code == qdec.QDEC_E_INVALID
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_prefill(0, [1, 2], 2, None, 0, 0)
    assert e.value.code == qdec.QDEC_E_INVALID
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_decode_step(0, 1, 0)
    assert e.value.code == qdec.QDEC_E_INVALID
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_decode_batch([], [])
    assert e.value.code == qdec.QDEC_E_INVALID
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_clone_state(0)
    assert e.value.code == qdec.QDEC_E_INVALID


def test_sample_rejects_without_model():
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_sample(0, None, 1, 1.0, 10, 1.0, 1.0, None, 0, [0.5], None)
    assert e.value.code == qdec.QDEC_E_INVALID


def test_batch_size_limit():
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_decode_batch([1] * 17, [0] * 17)
    assert e.value.code == qdec.QDEC_E_INVALID


def adaptor_cfg(**kw):
    base = dict(enc_dim=512, mid_dim=2048, dim=1024, ffn_dim=256, n_block=2, n_head=8, ln_eps=1e-12,
                weight_dtype=qdec.QDEC_BF16)
    base.update(kw)
    return qdec.qdec_adaptor_config(**base)


ADAPTOR_BAD = [dict(weight_dtype=qdec.QDEC_F32), dict(enc_dim=100), dict(mid_dim=2000), dict(ffn_dim=200),
               dict(dim=1000), dict(n_head=4), dict(n_block=0), dict(n_block=9), dict(ln_eps=0.0)]


@pytest.mark.parametrize("kw", ADAPTOR_BAD, ids=[str(k) for k in ADAPTOR_BAD])
def test_adaptor_create_rejects_bad_config(kw):
    w = qdec.qdec_adaptor_weights(0, 0, 0, 0, None)
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_adaptor_create(adaptor_cfg(**kw), w, 0)
    assert e.value.code == qdec.QDEC_E_INVALID


def test_adaptor_null_arguments():
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_adaptor_create(adaptor_cfg(), qdec.qdec_adaptor_weights(0, 0, 0, 0, None), 0)
    assert e.value.code == qdec.QDEC_E_INVALID  # weights incomplete
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_adaptor_run(0, 0, 4, 0)
    assert e.value.code == qdec.QDEC_E_INVALID
    qdec.qdec_adaptor_destroy(0)  # NULL is a no-op


def encoder_cfg(**kw):
    base = dict(n_mels=80, lfr_m=7, lfr_n=6, dim=512, n_head=4, ffn_dim=2048, fsmn_kernel=11, n_main=49, n_tp=20,
                ln_eps=1e-12, weight_dtype=qdec.QDEC_BF16)
    base.update(kw)
    return qdec.qdec_encoder_config(**base)


ENCODER_BAD = [dict(weight_dtype=qdec.QDEC_F32), dict(n_mels=64), dict(lfr_m=6), dict(lfr_m=17), dict(lfr_n=0),
               dict(dim=500), dict(n_head=3), dict(ffn_dim=1000), dict(fsmn_kernel=10), dict(fsmn_kernel=33),
               dict(n_main=-1), dict(n_tp=128), dict(ln_eps=0.0)]


@pytest.mark.parametrize("kw", ENCODER_BAD, ids=[str(k) for k in ENCODER_BAD])
def test_encoder_create_rejects_bad_config(kw):
    w = qdec.qdec_encoder_weights(None, 0, 0, 0, 0)
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_encoder_create(encoder_cfg(**kw), w, 0)
    assert e.value.code == qdec.QDEC_E_INVALID


def test_encoder_null_arguments_and_row_count():
    with pytest.raises(qdec.QdecError) as e:
        qdec.qdec_encoder_create(encoder_cfg(), qdec.qdec_encoder_weights(None, 0, 0, 0, 0), 0)
    assert e.value.code == qdec.QDEC_E_INVALID and "weights" in qdec.qdec_last_error()
    for call in (lambda: qdec.qdec_encoder_run(0, 0, 16000, 0), lambda: qdec.qdec_frontend_run(0, 0, 16000, 0),
                 lambda: qdec.qdec_encoder_forward(0, 0, 4, 0)):
        with pytest.raises(qdec.QdecError) as e:
            call()
        assert e.value.code == qdec.QDEC_E_INVALID
    assert qdec.qdec_encoder_rows(0, 16000) == 0  # NULL encoder
    qdec.qdec_encoder_destroy(0)  # NULL is a no-op
