"""C-ABI checks that need no GPU: the library loads, exports every function
include/mtp.h declares, and rejects bad arguments on the host before anything
is enqueued (so these calls never reach the HIP runtime)."""
import ctypes as C
import os
import re

import pytest

import mtp_speculative_draft_amd as mtp

FAKE = 0x100000  # a 256-aligned non-null address; never dereferenced by rejected calls


def _declared():
    text = open(mtp.HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mtp_[a-z0-9_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    names = _declared()
    assert len(names) >= 17
    lib = mtp.lib()
    for n in names:
        assert hasattr(lib, n), n
        assert n in mtp._SIGS, f"binding lacks {n}"


def test_status_strings_and_version():
    lib = mtp.lib()
    assert lib.mtp_status_string(0) == b"ok"
    assert lib.mtp_status_string(3) == b"workspace too small"
    assert b"gfx950" in lib.mtp_version()


def _q4(n=64, k=64, codes=FAKE, scales=FAKE, biases=FAKE):
    return mtp.MtpQ4(codes, scales, biases, n, k)


@pytest.mark.parametrize("m", [0, -1, 9])
def test_qgemv_rejects_row_counts(m):
    w = _q4()
    assert mtp.lib().mtp_qgemv(C.byref(w), FAKE, None, FAKE + 4096, m, None) == mtp.MTP_ERR_INVALID_ARG
    assert b"m=" in mtp.lib().mtp_last_error()


@pytest.mark.parametrize("n,k,codes,want", [
    (64, 48, FAKE, mtp.MTP_ERR_INVALID_ARG),       # k not a multiple of 32
    (0, 64, FAKE, mtp.MTP_ERR_INVALID_ARG),        # empty output
    (64, 8224, FAKE, mtp.MTP_ERR_UNSUPPORTED),     # k above the maximum
    (64, 64, FAKE + 8, mtp.MTP_ERR_INVALID_ARG),   # codes not 16-byte aligned
    (64, 64, None, mtp.MTP_ERR_INVALID_ARG),       # NULL codes
])
def test_qgemv_rejects_bad_weights(n, k, codes, want):
    w = _q4(n, k, codes=codes)
    assert mtp.lib().mtp_qgemv(C.byref(w), FAKE, None, FAKE + 4096, 1, None) == want


def test_qgemv_rejects_null_and_aliasing():
    w = _q4()
    lib = mtp.lib()
    assert lib.mtp_qgemv(None, FAKE, None, FAKE, 1, None) == mtp.MTP_ERR_INVALID_ARG
    assert lib.mtp_qgemv(C.byref(w), None, None, FAKE, 1, None) == mtp.MTP_ERR_INVALID_ARG
    assert lib.mtp_qgemv(C.byref(w), FAKE, None, FAKE, 1, None) == mtp.MTP_ERR_INVALID_ARG  # y aliases x
    assert lib.mtp_qgemv(C.byref(w), FAKE + 4, None, FAKE + 4096, 1, None) == mtp.MTP_ERR_INVALID_ARG


def _layer(H=256, nh=2, nkv=1, d=128, vocab=1000, inter=512):
    q = lambda n, k: _q4(n, k)  # noqa: E731
    z8 = mtp.MtpQ8(None, None, 0, 0, 0)
    return mtp.MtpLayer(H, nh, nkv, d, vocab, mtp.MTP_FFN_DENSE_Q4, inter, 0, 1e6, 1e-6,
                        FAKE, FAKE, FAKE, FAKE, FAKE,
                        q(H, 2 * H), q(nh * d, H), q(nkv * d, H), q(nkv * d, H), q(H, nh * d),
                        q(inter, H), q(inter, H), q(H, inter), q(vocab, H), None, z8, z8, z8, z8, z8, z8)


def test_workspace_sizes_are_host_arithmetic():
    lib = mtp.lib()
    L = _layer()
    a1 = lib.mtp_attn_decode_workspace_size(C.byref(L), 4096, 1)
    a4 = lib.mtp_attn_decode_workspace_size(C.byref(L), 4096, 4)
    assert 0 < a1 < a4
    assert lib.mtp_ffn_dense_workspace_size(6144, 4) >= 4 * 6144 * 4
    assert lib.mtp_lmhead_workspace_size(151936, 1) > 0
    d = lib.mtp_draft_step_workspace_size(C.byref(L), 4096, 4)
    assert d > a4
    assert lib.mtp_ffn_moe_workspace_size(2048, 256, 8, 512, 512, 4) >= 33 * 4 * 2048 * 4
    assert lib.mtp_ffn_dense_workspace_size(0, 1) == 0


def test_draft_step_rejects_cache_overflow_and_small_workspace():
    lib = mtp.lib()
    L = _layer()
    need = lib.mtp_draft_step_workspace_size(C.byref(L), 10, 4)
    args = lambda cache_len, cap, ws_bytes: (C.byref(L), FAKE, None, None, FAKE, FAKE * 2, FAKE * 3, cache_len,  # noqa: E731
                                             cap, 4, FAKE * 4, FAKE * 5, None, FAKE * 6, ws_bytes, None)
    assert lib.mtp_draft_step(*args(10, 13, need)) == mtp.MTP_ERR_INVALID_ARG
    assert b"overflow" in lib.mtp_last_error()
    assert lib.mtp_draft_step(*args(10, 14, need - 1)) == mtp.MTP_ERR_WORKSPACE
    assert lib.mtp_draft_step(*args(-1, 14, need)) == mtp.MTP_ERR_INVALID_ARG


def test_attention_rejects_unsupported_head_dim_and_bad_group():
    lib = mtp.lib()
    L = _layer(d=64)
    assert lib.mtp_attn_decode(C.byref(L), FAKE, FAKE * 2, FAKE * 3, 0, 16, 1, FAKE * 4, FAKE * 5, 1 << 30,
                               None) == mtp.MTP_ERR_UNSUPPORTED
    L = _layer(nh=3, nkv=2)
    assert lib.mtp_attn_decode(C.byref(L), FAKE, FAKE * 2, FAKE * 3, 0, 16, 1, FAKE * 4, FAKE * 5, 1 << 30,
                               None) == mtp.MTP_ERR_INVALID_ARG


def test_moe_rejects_bad_top_k_and_half_given_shared_expert():
    lib = mtp.lib()
    g = mtp.MtpQ8(FAKE, FAKE, 64, 64, 4)
    d = mtp.MtpQ8(FAKE, FAKE, 64, 64, 4)
    call = lambda k, sg: lib.mtp_ffn_moe_q(FAKE, None, 1e-6, FAKE, k, C.byref(g), C.byref(g), C.byref(d),  # noqa: E731
                                           sg, None, None, None, FAKE * 2, None, None, 1, FAKE * 3, 1 << 30, None)
    assert call(5, None) == mtp.MTP_ERR_INVALID_ARG
    assert call(0, None) == mtp.MTP_ERR_INVALID_ARG
    assert call(2, C.byref(g)) == mtp.MTP_ERR_INVALID_ARG


def test_lmhead_requires_ids_and_workspace():
    lib = mtp.lib()
    w = _q4(1000, 256)
    assert lib.mtp_lmhead_argmax(FAKE, FAKE, 1e-6, C.byref(w), None, None, None, 1, FAKE, 1 << 20,
                                 None) == mtp.MTP_ERR_INVALID_ARG
    assert lib.mtp_lmhead_argmax(FAKE, FAKE, 1e-6, C.byref(w), None, None, FAKE * 2, 1, FAKE * 3, 16,
                                 None) == mtp.MTP_ERR_WORKSPACE


def test_layer_struct_layout_matches_the_header(tmp_path):
    """The binding's mtp_layer mirrors include/mtp.h field for field."""
    import subprocess
    src = tmp_path / "layout.c"
    fields = ("sh_down", "gamma_q_head", "q_gated", "rotary_dim", "sinks", "window", "v_head_dim", "gate_exps4",
              "sh_down4", "mrope_section", "positions")
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "mtp.h"\n'
                   'int main(void) { printf("%zu %zu\\n", sizeof(mtp_layer), sizeof(mtp_q4e));'
                   + "".join(f' printf("%zu\\n", offsetof(mtp_layer, {f}));' for f in fields)
                   + ' return 0; }\n')
    exe = tmp_path / "layout"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.dirname(mtp.HEADER), str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    L = mtp.MtpLayer
    assert got == [C.sizeof(L), C.sizeof(mtp.MtpQ4E)] + [getattr(L, f).offset for f in fields]


def test_attention_variant_fields_are_validated():
    lib = mtp.lib()

    def status(L):
        return lib.mtp_attn_decode(C.byref(L), FAKE, FAKE * 2, FAKE * 3, 0, 16, 1, FAKE * 4, FAKE * 5, 1 << 30, None)

    L = _layer()
    L.rotary_dim = 48  # not a power of two
    assert status(L) == mtp.MTP_ERR_UNSUPPORTED
    L = _layer()
    L.rotary_dim = 256  # above head_dim
    assert status(L) == mtp.MTP_ERR_UNSUPPORTED
    L = _layer()
    L.q_gated = 1  # wq still has n_heads * head_dim rows
    assert status(L) == mtp.MTP_ERR_INVALID_ARG
    L = _layer()
    L.gamma_q_head = FAKE  # without gamma_k_head
    assert status(L) == mtp.MTP_ERR_INVALID_ARG
    assert b"gamma_k_head" in lib.mtp_last_error()
    L = _layer()
    L.window = -1
    assert status(L) == mtp.MTP_ERR_INVALID_ARG
    assert b"window" in lib.mtp_last_error()
    L = _layer()
    L.sinks = FAKE + 2  # not 4-byte aligned
    assert status(L) == mtp.MTP_ERR_INVALID_ARG
    assert b"sinks" in lib.mtp_last_error()
    L = _layer()
    L.head_dim = 192  # V heads of 192 are not built
    assert status(L) == mtp.MTP_ERR_UNSUPPORTED
    L = _layer()
    L.v_head_dim = 64
    assert status(L) == mtp.MTP_ERR_UNSUPPORTED
    L = _layer()
    L.v_head_dim = -1
    assert status(L) == mtp.MTP_ERR_INVALID_ARG


def test_append_kv_rejects_overflow_and_empty_batches():
    lib = mtp.lib()
    L = _layer()
    need = lib.mtp_append_kv_workspace_size(C.byref(L))
    assert need > 0
    args = lambda cache_len, cap, m, ws_bytes: (C.byref(L), FAKE, None, None, None, FAKE * 2, FAKE * 3, FAKE * 4,  # noqa: E731
                                                cache_len, cap, m, FAKE * 5, ws_bytes, None)
    assert lib.mtp_append_kv(*args(10, 13, 4, need)) == mtp.MTP_ERR_INVALID_ARG
    assert b"overflow" in lib.mtp_last_error()
    assert lib.mtp_append_kv(*args(10, 14, 0, need)) == mtp.MTP_ERR_INVALID_ARG
    assert lib.mtp_append_kv(*args(10, 14, 4, need - 1)) == mtp.MTP_ERR_WORKSPACE


def test_accept_is_the_longest_matching_prefix_and_records_the_round():
    st = mtp.MtpStats()
    assert mtp.mtp_accept([5, 7, 9], [5, 7, 9, 11], st) == 3  # all drafts accepted, 11 is the bonus token
    assert mtp.mtp_accept([5, 7, 9], [5, 8, 9, 11], st) == 1  # a later match after a miss does not count
    assert mtp.mtp_accept([5, 7, 9], [4, 7, 9, 11], st) == 0
    assert mtp.mtp_accept([1], [1, 2], st) == 1
    assert (st.rounds, st.drafted, st.accepted) == (4, 10, 5)
    assert list(st.accept_hist)[:4] == [1, 2, 0, 1]
    assert list(st.depth_drafted)[:3] == [4, 3, 3] and list(st.depth_accepted)[:3] == [3, 1, 1]
    lib = mtp.lib()
    arr = (C.c_int32 * 20)()
    assert lib.mtp_accept(arr, arr, 0, None) == -1
    assert lib.mtp_accept(arr, arr, mtp.MTP_MAX_DRAFT + 1, None) == -1
    assert lib.mtp_accept(None, arr, 2, None) == -1
    assert mtp.mtp_accept([3, 3], [3, 3, 0]) == 2  # stats are optional


def test_stats_struct_layout_matches_the_header(tmp_path):
    import subprocess
    src = tmp_path / "stats.c"
    src.write_text('#include <stddef.h>\n#include <stdio.h>\n#include "mtp.h"\n'
                   'int main(void) { printf("%zu %zu %zu\\n", sizeof(mtp_stats), offsetof(mtp_stats, accept_hist), '
                   'offsetof(mtp_stats, depth_accepted)); return 0; }\n')
    exe = tmp_path / "stats"
    subprocess.check_call(["gcc", "-std=c99", "-I", os.path.dirname(mtp.HEADER), str(src), "-o", str(exe)])
    got = [int(v) for v in subprocess.check_output([str(exe)]).split()]
    S = mtp.MtpStats
    assert got == [C.sizeof(S), S.accept_hist.offset, S.depth_accepted.offset]


def test_stack_draft_rejects_bad_layers():
    lib = mtp.lib()
    L = _layer()
    arr = (mtp.MtpStackLayer * 2)()
    arr[0] = mtp.MtpStackLayer(C.addressof(L), FAKE, FAKE * 2, 64, 5)
    arr[1] = mtp.MtpStackLayer(C.addressof(L), FAKE * 3, FAKE * 4, 64, 11)  # start past t
    ws = lib.mtp_stack_draft_workspace_size(arr, 2, 10)
    assert ws > 0
    assert lib.mtp_stack_draft(arr, 2, FAKE * 5, FAKE * 6, FAKE * 7, 10, FAKE * 8, ws, None) == mtp.MTP_ERR_INVALID_ARG
    arr[1].start = 3
    arr[1].capacity = 10  # row t = 10 beyond capacity
    assert lib.mtp_stack_draft(arr, 2, FAKE * 5, FAKE * 6, FAKE * 7, 10, FAKE * 8, ws, None) == mtp.MTP_ERR_INVALID_ARG
    assert lib.mtp_stack_draft(arr, 0, FAKE * 5, FAKE * 6, FAKE * 7, 10, FAKE * 8, ws, None) == mtp.MTP_ERR_INVALID_ARG


def _gpu_visible():
    try:
        import torch
        return torch.cuda.device_count() > 0  # counts devices without initialising them
    except Exception:
        return False


@pytest.mark.skipif(_gpu_visible(), reason="passes fake device pointers; a check that failed to reject would launch them")
def test_stack_draft_checks_every_layer_before_launching():
    """A valid layer 0 and a layer 1 without a K cache: the call must fail in
    its checks (MTP_ERR_INVALID_ARG), before layer 0's catch-up or draft is
    enqueued (with no device here, any launch would surface as MTP_ERR_HIP)."""
    lib = mtp.lib()
    L = _layer()
    arr = (mtp.MtpStackLayer * 2)()
    arr[0] = mtp.MtpStackLayer(C.addressof(L), FAKE, FAKE * 2, 64, 5)
    arr[1] = mtp.MtpStackLayer(C.addressof(L), None, FAKE * 4, 64, 5)
    ws = lib.mtp_stack_draft_workspace_size(arr, 2, 10)
    assert lib.mtp_stack_draft(arr, 2, FAKE * 5, FAKE * 6, FAKE * 7, 10, FAKE * 8, ws, None) == mtp.MTP_ERR_INVALID_ARG
    assert b"layer 1" in lib.mtp_last_error()
    # a bad workspace size is caught the same way (no partial work for layer 0)
    arr[1].k_cache = FAKE * 3
    assert lib.mtp_stack_draft(arr, 2, FAKE * 5, FAKE * 6, FAKE * 7, 10, FAKE * 8, ws - 256, None) in (
        mtp.MTP_ERR_WORKSPACE, mtp.MTP_ERR_INVALID_ARG)


def test_token_rows_need_a_vocabulary():
    lib = mtp.lib()
    L = _layer(vocab=0)
    need = lib.mtp_append_kv_workspace_size(C.byref(L))
    assert lib.mtp_append_kv(C.byref(L), None, FAKE, FAKE * 2, None, FAKE * 3, FAKE * 4, FAKE * 5, 0, 16, 2,
                             FAKE * 6, need, None) == mtp.MTP_ERR_INVALID_ARG
    assert b"vocab" in lib.mtp_last_error()


def test_every_workspace_reserves_the_argmax_state():
    """The first 1152 bytes of every workspace belong to the head's argmax
    state, so every size covers at least them plus one 256-byte piece."""
    lib = mtp.lib()
    L = _layer()
    assert lib.mtp_lmhead_workspace_size(1000, 1) == 1152
    for n in (lib.mtp_attn_decode_workspace_size(C.byref(L), 10, 1), lib.mtp_ffn_dense_workspace_size(64, 1),
              lib.mtp_append_kv_workspace_size(C.byref(L)), lib.mtp_draft_step_workspace_size(C.byref(L), 10, 1),
              lib.mtp_ffn_moe_workspace_size(256, 16, 4, 64, 64, 1)):
        assert n >= 1280 + 256


def test_noalloc_draft_step_rejects_steps_beyond_its_scratch():
    """The allocation-free draft step runs every argument check, then rejects a
    step whose workspace would exceed the static scratch, before any HIP call
    (no GPU here: reaching the runtime would give MTP_ERR_HIP instead)."""
    lib = mtp.lib()
    L = _layer()
    big = 1 << 22
    assert lib.mtp_draft_step_workspace_size(C.byref(L), big, 8) > mtp.MTP_NOALLOC_SCRATCH_BYTES
    args = lambda cache_len, cap, m: (C.byref(L), FAKE, None, None, FAKE, FAKE * 2, FAKE * 3, cache_len,  # noqa: E731
                                      cap, m, FAKE * 4, FAKE * 5, None, None)
    assert lib.mtp_draft_step_noalloc(*args(big, big + 8, 8)) == mtp.MTP_ERR_WORKSPACE
    msg = lib.mtp_last_error()
    assert b"MTP_NOALLOC_SCRATCH_BYTES" in msg and b"mtp_draft_step with a workspace" in msg
    # argument errors come first and read as those of mtp_draft_step
    assert lib.mtp_draft_step_noalloc(*args(big, big + 7, 8)) == mtp.MTP_ERR_INVALID_ARG
    assert b"overflow" in lib.mtp_last_error()
    assert lib.mtp_draft_step_noalloc(*args(10, 20, 9)) == mtp.MTP_ERR_INVALID_ARG


def test_moe_q4_rejects_unbuilt_shapes_and_mixed_formats():
    """4-bit experts run on the slot kernel only: other feature counts, or a
    shared expert of another size, are MTP_ERR_UNSUPPORTED; bad descriptors
    are rejected before anything is enqueued."""
    lib = mtp.lib()
    q = lambda n, k, E=4: mtp.MtpQ4E(FAKE, FAKE, FAKE, n, k, E)  # noqa: E731
    ws_big = 1 << 30

    def call(ge, ue, de, sh=(None, None, None), H=None, top_k=2):
        return lib.mtp_ffn_moe_q4(FAKE, None, 1e-6, FAKE, top_k, C.byref(ge), C.byref(ue), C.byref(de),
                                  *(None if w is None else C.byref(w) for w in sh), None, FAKE * 2, None, None, 1,
                                  FAKE * 3, ws_big, None)
    assert call(q(96, 2048), q(96, 2048), q(2048, 96)) == mtp.MTP_ERR_UNSUPPORTED  # inter 96: 3 groups
    assert b"4-bit experts" in lib.mtp_last_error()
    assert call(q(512, 1024), q(512, 1024), q(1024, 512)) == mtp.MTP_ERR_UNSUPPORTED  # hidden 1024: 32 groups
    sh = (q(256, 2048, 1), q(256, 2048, 1), q(2048, 256, 1))
    assert call(q(512, 2048), q(512, 2048), q(2048, 512), sh) == mtp.MTP_ERR_UNSUPPORTED
    assert b"shared expert" in lib.mtp_last_error()
    bad = mtp.MtpQ4E(FAKE, FAKE, None, 512, 2048, 4)  # no biases
    assert call(bad, q(512, 2048), q(2048, 512)) == mtp.MTP_ERR_INVALID_ARG
    odd = mtp.MtpQ4E(FAKE, FAKE + 1, FAKE, 512, 2048, 4)  # bf16 scales must be 2-byte aligned
    assert call(odd, q(512, 2048), q(2048, 512)) == mtp.MTP_ERR_INVALID_ARG
    assert call(q(512, 2048), q(512, 2048), q(2048, 512, 3)) == mtp.MTP_ERR_INVALID_ARG  # expert counts differ
    assert lib.mtp_dequant_q4e(C.byref(q(512, 2048)), 4, FAKE, None) == mtp.MTP_ERR_INVALID_ARG


def test_draft_step_takes_the_4bit_expert_layer_fields():
    """ffn_kind MTP_FFN_MOE_Q4 reads gate_exps4 ... sh_down4: a layer whose
    4-bit stacks are missing is rejected, and its workspace is sized from them."""
    lib = mtp.lib()
    L = _layer(H=2048)
    L.ffn_kind = mtp.MTP_FFN_MOE_Q4
    L.top_k = 2
    L.router = FAKE
    args = (C.byref(L), FAKE, None, None, FAKE, FAKE * 2, FAKE * 3, 10, 20, 1, FAKE * 4, FAKE * 5, None, FAKE * 6,
            1 << 30, None)
    assert lib.mtp_draft_step(*args) == mtp.MTP_ERR_INVALID_ARG
    assert b"gate_exps" in lib.mtp_last_error()
    a = lib.mtp_draft_step_workspace_size(C.byref(L), 10, 4)
    L.gate_exps4 = mtp.MtpQ4E(FAKE, FAKE, FAKE, 512, 2048, 256)
    assert lib.mtp_draft_step_workspace_size(C.byref(L), 10, 4) > a


def test_rotary_positions_are_validated():
    """Negative section sizes, misaligned position ids and position ids on the
    head-192 geometry are rejected on the host."""
    lib = mtp.lib()
    need = 1 << 30
    args = lambda L: (C.byref(L), FAKE, FAKE * 2, FAKE * 3, 10, 20, 1, FAKE * 4, FAKE * 5, need, None)  # noqa: E731
    L = _layer()
    L.mrope_section[1] = -1
    assert lib.mtp_attn_decode(*args(L)) == mtp.MTP_ERR_INVALID_ARG
    assert b"mrope_section" in lib.mtp_last_error()
    L = _layer()
    L.positions = FAKE + 2
    assert lib.mtp_attn_decode(*args(L)) == mtp.MTP_ERR_INVALID_ARG
    assert b"positions" in lib.mtp_last_error()
    L = _layer(d=192)
    L.v_head_dim = 128
    L.wq = _q4(2 * 192, 256)
    L.wk = _q4(192, 256)
    L.wv = _q4(128, 256)
    L.wo = _q4(256, 2 * 128)
    L.positions = FAKE
    assert lib.mtp_attn_decode(*args(L)) == mtp.MTP_ERR_UNSUPPORTED
    assert b"positions" in lib.mtp_last_error()
