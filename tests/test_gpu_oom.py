"""QDEC_E_OOM on a live GPU (include/qdec.h, "Errors"). The environment
variable QDEC_DEVICE_LIMIT_BYTES caps the device bytes the library holds, so
each allocation path fails as it would on a full HBM while the GPU still has
room for everything else. Every such failure must return QDEC_E_OOM, hand
back no object, leave the state where it was, and the same call must succeed
once the cap is lifted, with logits that still match the oracle (tiny fp32
decoder, 1e-4). Calls that allocate nothing (a decode step after prefill,
the no-alloc sampler) must keep working under a one-byte cap."""
import numpy as np
import pytest

import oracle
import synth

from .gpu_harness import device_model, torch_dev

pytestmark = pytest.mark.gpu

LIMIT = "QDEC_DEVICE_LIMIT_BYTES"


def _oom(fn, *args, what):
    from qwen3_kv_cache_amd import qdec
    with pytest.raises(qdec.QdecError) as e:
        fn(*args)
    assert e.value.code == qdec.QDEC_E_OOM, (e.value.code, qdec.qdec_last_error())
    assert what in qdec.qdec_last_error(), qdec.qdec_last_error()


def test_decoder_allocation_failures(monkeypatch):
    from qwen3_kv_cache_amd import qdec
    w = synth.WORKLOADS["tiny"]
    W = synth.make_weights(w.shape, w.weight_seed)
    ids, audio, a0 = synth.make_prompt(w)
    T, V = len(ids), w.shape.vocab
    orc = oracle.Qwen3Oracle(oracle.OracleConfig.from_shape(w.shape), W.f32)
    toks, ref = oracle.greedy_trajectory(orc, ids, audio, a0, 2)
    torch, dev = torch_dev()

    print("[oom] create", flush=True)
    monkeypatch.setenv(LIMIT, "0")
    _oom(device_model, w.shape, W, what="packed weights")
    monkeypatch.delenv(LIMIT)
    m = device_model(w.shape, W)
    big = st = None
    try:
        # a 4096-position state leaves the KV pool without a free page
        big = qdec.qdec_state_create(m.handle, 4096)
        print("[oom] state", flush=True)
        monkeypatch.setenv(LIMIT, "1")
        _oom(qdec.qdec_state_create, m.handle, T + 2, what="KV pool")
        monkeypatch.delenv(LIMIT)
        st = qdec.qdec_state_create(m.handle, T + 2)
        qdec.qdec_state_destroy(big)
        big = None

        audio_d = torch.from_numpy(audio).to(dev)
        ap = audio_d.data_ptr()
        lg = torch.full((3, V), float("nan"), dtype=torch.float32, device=dev)
        am = torch.full((3,), -1, dtype=torch.int32, device=dev)
        print("[oom] prefill", flush=True)
        monkeypatch.setenv(LIMIT, "1")
        _oom(qdec.qdec_prefill, st, ids, T, ap, a0, len(audio), lg[0].data_ptr(), am[0].data_ptr(),
             what="prefill")
        assert qdec.qdec_state_pos(st) == 0
        monkeypatch.delenv(LIMIT)
        qdec.qdec_prefill(st, ids, T, ap, a0, len(audio), lg[0].data_ptr(), am[0].data_ptr())

        print("[oom] decode step under a one-byte cap", flush=True)
        monkeypatch.setenv(LIMIT, "1")
        qdec.qdec_decode_step(st, int(toks[0]), T, lg[1].data_ptr(), am[1].data_ptr())
        assert qdec.qdec_state_pos(st) == T + 1

        print("[oom] batch", flush=True)
        _oom(qdec.qdec_decode_batch, [st], [int(toks[1])], lg[2].data_ptr(), am[2].data_ptr(), what="batch")
        assert qdec.qdec_state_pos(st) == T + 1
        monkeypatch.delenv(LIMIT)
        qdec.qdec_decode_batch([st], [int(toks[1])], lg[2].data_ptr(), am[2].data_ptr())
        assert qdec.qdec_state_pos(st) == T + 2

        print("[oom] sampling", flush=True)
        tok_a = torch.full((1,), -1, dtype=torch.int32, device=dev)
        tok_b = torch.full((1,), -1, dtype=torch.int32, device=dev)
        args = (lg[2].data_ptr(), 1, 0.8, 20, 0.9, 1.0, None, 0, [0.37])
        monkeypatch.setenv(LIMIT, "1")
        _oom(qdec.qdec_sample, m.handle, *args, tok_a.data_ptr(), what="sampling")
        qdec.qdec_sample_noalloc(m.handle, *args, tok_b.data_ptr())
        monkeypatch.delenv(LIMIT)
        qdec.qdec_sample(m.handle, *args, tok_a.data_ptr())
        torch.cuda.synchronize()

        got = lg.cpu().numpy()
        err = float(np.max(np.abs(got - ref)))
        assert err <= 1e-4, f"max |gpu - oracle| = {err}"
        assert list(am.cpu().numpy()) == list(toks[:3])
        assert int(tok_a.item()) == int(tok_b.item()) and 0 <= int(tok_a.item()) < V
    finally:
        monkeypatch.delenv(LIMIT, raising=False)
        if big:
            qdec.qdec_state_destroy(big)
        if st:
            qdec.qdec_state_destroy(st)
        m.close()


def test_adaptor_and_encoder_allocation_failures(monkeypatch):
    from qwen3_kv_cache_amd.device import Adaptor, Encoder
    torch, dev = torch_dev()
    print("[oom] adaptor create", flush=True)
    shape = synth.AdaptorShape(n_block=1)
    _, bits = synth.make_adaptor_weights(shape, 27)
    monkeypatch.setenv(LIMIT, "0")
    _oom(Adaptor, shape, bits, what="adaptor")
    monkeypatch.delenv(LIMIT)
    a = Adaptor(shape, bits)
    try:
        frames = torch.randn((40, shape.enc_dim), dtype=torch.float32, device=dev)
        want = a.run(frames).cpu().numpy()
        # a longer input needs larger scratch
        long = torch.randn((400, shape.enc_dim), dtype=torch.float32, device=dev)
        monkeypatch.setenv(LIMIT, "1")
        _oom(a.run, long, what="adaptor")
        monkeypatch.delenv(LIMIT)
        got = a.run(frames).cpu().numpy()
        assert np.array_equal(got, want)
        assert np.all(np.isfinite(a.run(long).cpu().numpy()))
    finally:
        monkeypatch.delenv(LIMIT, raising=False)
        a.close()

    print("[oom] encoder", flush=True)
    eshape = synth.EncoderShape(n_main=1, n_tp=0)
    _, ebits = synth.make_encoder_weights(eshape, 1)
    monkeypatch.setenv(LIMIT, "0")
    _oom(Encoder, eshape, ebits, what="encoder")
    monkeypatch.delenv(LIMIT)
    e = Encoder(eshape, ebits)
    try:
        short = torch.from_numpy(synth.pcm("voiced", 16000, 5)).to(dev)
        want = e.run(short).cpu().numpy()
        long = torch.from_numpy(synth.pcm("voiced", 64000, 5)).to(dev)
        monkeypatch.setenv(LIMIT, "1")
        _oom(e.run, long, what="fbank")
        monkeypatch.delenv(LIMIT)
        assert np.array_equal(e.run(short).cpu().numpy(), want)
        assert np.all(np.isfinite(e.run(long).cpu().numpy()))
    finally:
        monkeypatch.delenv(LIMIT, raising=False)
        e.close()
