"""Shapes that together reach every kernel variant the host dispatch can
choose, at every head dimension.  The CPU suite checks the coverage through
the plan query (no GPU needed); the GPU suite runs each shape against the
oracle.  Entries: (name, (batch, n_h, n_kv_h, T, s_k), split_len (0 =
fmha_forward), causal, window)."""

SHAPES = [
    ("one-slice-streamed-small", (2, 4, 2, 3, 50), 0, True, 0),
    ("one-slice-shared-small", (2, 8, 1, 5, 50), 0, False, 0),
    ("multi-few-units", (2, 8, 2, 20, 300), 0, True, 0),
    ("one-slice-streamed-split", (4, 8, 8, 1, 2048), 32, False, 0),
    ("one-slice-shared-split", (4, 32, 2, 2, 1024), 32, True, 0),
    ("multi-one-tile", (8, 64, 64, 1, 700), 0, True, 300),
    ("multi-two-tiles", (32, 16, 8, 20, 300), 0, True, 0),
    ("row-parallel-gqa", (4, 64, 32, 100, 300), 0, True, 0),
    ("row-parallel-window", (4, 64, 64, 100, 300), 0, True, 70),
    ("row-parallel-two-tiles", (4, 128, 128, 100, 200), 0, True, 0),
    ("mqa-short-cache", (2, 32, 1, 1, 100), 0, False, 0),
    ("window-group7-straddling-tiles", (1, 7, 1, 40, 300), 0, True, 30),
    ("wide-streamed-256", (2, 4, 4, 1, 250), 0, True, 0),
    ("wide-shared-512", (2, 40, 1, 1, 500), 0, False, 0),
    ("wide-streamed-split-512", (2, 8, 2, 3, 1300), 480, True, 0),
    ("wide-shared-split-256", (1, 48, 2, 1, 700), 200, False, 0),
    ("multi-eight-waves", (40, 128, 1, 1, 300), 0, False, 0),
    ("one-pass-shared-split", (2, 32, 1, 1, 256), 128, False, 0),
]

HEAD_DIMS = (64, 128, 256, 512)


def branch(plan: dict) -> str:
    """The kernel variant a plan launches: the kernel template instance with
    its output mode (fused or split) left out."""
    family, args = plan["kernel"].split("<", 1)
    args = args.rstrip(">").split(", ")
    del args[_SPLIT_ARG[family]]
    return f"{family}<{', '.join(args)}>"


# every variant the dispatcher launches at a head dimension (at hd 128 the
# split decode falls back to the per-wave one-slice kernels only when the
# stream kernel's 32-bit partial offsets do not reach -- 2^18 partition slots
# for one 16-row tile; test_split_decode_with_partition_slots_past_the_
# stream_kernel_offsets covers that case)
EXPECTED = {
    64: {"attn_kernel<64, 4, 4, 1, 1, false, false>", "attn_kernel<64, 4, 4, 1, 2, false, false>",
         "attn_kernel<64, 4, 4, 1, 1, true, false>", "attn_kernel<64, 4, 4, 1, 1, true, true>",
         "stream_kernel<64, true, 8, 1>", "stream_kernel<64, false, 8, 1>",
         "stream_kernel<64, true, 8, 2>", "stream_kernel<64, false, 8, 2>",
         "rows_kernel<64, 1, 64>", "rows_kernel<64, 2, 32>"},
    128: {"attn_kernel<128, 4, 4, 1, 1, false, false>", "attn_kernel<128, 4, 4, 1, 2, false, false>",
          "stream_kernel<128, true, 4, 1>", "stream_kernel<128, false, 4, 1>",
          "stream_kernel<128, true, 8, 1>", "stream_kernel<128, false, 8, 1>",
          "stream_kernel<128, true, 8, 2>", "stream_kernel<128, false, 8, 2>",
          "rows_kernel<128, 1, 64>", "rows_kernel<128, 2, 32>"},
    256: {"attn_kernel<256, 4, 2, 2, 1, false, false>", "attn_kernel<256, 4, 2, 2, 2, false, false>",
          "attn_kernel<256, 8, 4, 2, 1, false, false>", "cols_kernel<256, false>", "pass_kernel<256>",
          "pass_loop_kernel<256>",
          "rows_kernel<256, 1, 32>"},
    512: {"attn_kernel<512, 4, 1, 4, 1, false, false>", "attn_kernel<512, 4, 1, 4, 2, false, false>",
          "attn_kernel<512, 8, 2, 4, 1, false, false>", "cols_kernel<512, false>", "cols_kernel<512, true>", "pass_loop_kernel<512>",
          "rows_split_kernel<512>"},
}


# position of the SPLIT template argument in each kernel family's name
_SPLIT_ARG = {"attn_kernel": 5, "rows_kernel": 3, "rows_split_kernel": 1, "stream_kernel": 1, "pass_kernel": 1,
              "pass_loop_kernel": 1, "cols_kernel": 1}


def split_twin(kernel: str) -> str:
    """The name of the split-output instance of a forward kernel instance:
    the same template arguments with SPLIT = true."""
    family, args = kernel.split("<", 1)
    args = args.rstrip(">").split(", ")
    i = _SPLIT_ARG[family]
    assert args[i] == "false", kernel
    args[i] = "true"
    return f"{family}<{', '.join(args)}>"


def same_variant(plan_fwd: dict, plan_split: dict) -> bool:
    """A forward plan and a split plan launch the same kernel variant (the
    same template arguments apart from the output mode)."""
    a = {k: v for k, v in plan_fwd.items() if k != "kernel"}
    b = {k: v for k, v in plan_split.items() if k != "kernel"}
    return a == b and split_twin(plan_fwd["kernel"]) == plan_split["kernel"]
