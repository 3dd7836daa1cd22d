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

// Enqueue the LDS bank probe on `stream`: `blocks` workgroups of one wave
// each repeat one LDS access `iters` times.  form: 0 ds_read_b32, 1
// ds_read_b64, 2 ds_read_b128, 3 ds_read2_b64 (second address 32 bytes on),
// 4 ds_read2_b32 (16 bytes on), 5 ds_write_b32, 6 ds_write_b64, 7
// ds_write_b128, 8 ds_write2_b32 (272 bytes on).  lane_offsets (host, 64
// ints): each lane's byte offset into a 64 KiB LDS array, 4-byte aligned and
// below 65216, or negative for a lane that stays inactive.  `sink` (device,
// blocks * 64 floats) receives one value per lane.  Returns 0, 1 for a bad
// argument, 4 if the launch failed.
__attribute__((visibility("default"))) int kda_calibrate_lds(int form, const int* lane_offsets, int blocks,
                                                            int iters, float* sink, void* stream);

#ifdef __cplusplus
}
#endif
