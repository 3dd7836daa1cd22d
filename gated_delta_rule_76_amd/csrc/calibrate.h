// Calibration entry points of libkda_calibrate.so (benchmark support, not
// part of the KDA library's C ABI in include/).
#pragma once

#ifdef __cplusplus
extern "C" {
#endif

// Threads per workgroup of the calibration kernels.
__attribute__((visibility("default"))) int kda_calibrate_threads_per_block(void);

// Flops one kda_calibrate_mfma launch performs (2 per multiply-add).
__attribute__((visibility("default"))) double kda_calibrate_flops(int kind, int blocks, int iters);

// Enqueue the dense bf16 MFMA loop on `stream`: kind 0 = 16x16x32
// instructions, kind 1 = 32x32x16; `blocks` workgroups each run `iters`
// iterations; `sink` (device, blocks * threads_per_block floats) receives one
// value per thread so the work is not optimised away.  Returns 0, 1 for a bad
// argument, 4 if the launch failed.
__attribute__((visibility("default"))) int kda_calibrate_mfma(int kind, int blocks, int iters,
                                                             float* sink, void* stream);

#ifdef __cplusplus
}
#endif
