"""MI355X-native implementation of TIDE's one-GPU hot path: the level-1
bf16 -> fp32 reduce-scatter into padded rank-major shards and the all-gather
placement into parameter storage (C ABI in include/tide.h, HIP kernels for
gfx950 in csrc/). Importing this package loads libtide.so and fails loudly if
it has not been built."""
from ._lib import (  # noqa: F401
    Call,
    ENGINE_KERNEL,
    ENGINE_RUNTIME,
    ENGINE_SDMA,
    ENGINES,
    EXPORTS,
    FLAG_NO_LDS_FENCE,
    FLAG_SCALAR_PATH,
    LAUNCH_BUDGETED,
    LAUNCH_FULL,
    LIB_PATH,
    Launch,
    Plan,
    PointerTable,
    TideError,
    allgather_place,
    allgather_place_stage,
    budgeted,
    counted,
    decode_trace,
    diag_occupy,
    dma_engine_count,
    grads_table,
    landing_sum_fp32,
    landing_trace_records,
    latin_square,
    lib,
    params_table,
    plan_create,
    prepare_allgather_place,
    prepare_reduce_scatter_bf16_fp32,
    prepare_stage_grads_bf16,
    rd_schedule,
    reduce_scatter_bf16_fp32,
    reduce_scatter_bf16_fp32_noalloc,
    slot_grads_table,
    stage_grads_bf16,
    trace_buffer,
    traced,
    version,
)

lib()  # load now: no silent fallback exists
