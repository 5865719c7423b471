// Launchers of the device kernels (implemented in kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "plan_types.h"

namespace gkv {

// Byte copy of n token rows (n_kv head rows of head_bytes each, a multiple
// of 16) into the COLD slots named by slots (dev), head g of a row into
// position cold_row_pos(g, slot, cold_mask_for(n_kv)) of its slot; slots
// outside [0, cold_cap) are skipped.
hipError_t launch_cold_append(const void* k_new, const void* v_new, const int32_t* slots,
                              int32_t n, void* k_cold, void* v_cold, int32_t n_kv, int64_t head_bytes,
                              int32_t cold_cap, hipStream_t stream);

// Scatter n token rows ([n][n_kv][head_dim]) into the blocked HOT layout,
// starting at pool token tok0 (a slab's offset plus the first row's index).
hipError_t launch_hot_write(const void* k_rows, const void* v_rows, int32_t n, int64_t tok0, int32_t n_kv,
                           int32_t head_dim, int32_t dtype, int64_t hot_blocks, void* k_hot, void* v_hot,
                           hipStream_t stream);

// The step kernel: prefix splits of the chosen backend, suffix parts and the
// in-kernel join of partials, in one launch.  With `ev` non-null the launch
// stamps ev[0] / ev[1] with the kernel's start and end.
hipError_t launch_step(const StepArgs& a, int32_t dtype, int32_t backend, hipStream_t stream,
                       hipEvent_t* ev = nullptr);

// Streaming read of `bytes` (a multiple of 16) at p with `workgroups`
// workgroups; the data is discarded (sink: dev, 4 bytes, normally untouched).
hipError_t launch_stream_read(const void* p, size_t bytes, int32_t workgroups, uint32_t* sink,
                              hipStream_t stream);

// Device address of the static scratch of the allocation-free step on
// `device` (which must be current), from hipGetSymbolAddress on its first
// use there; *first_use tells the caller to clear what must start at zero.
hipError_t scratch_region(int device, uint8_t** ptr, bool* first_use);

// Zeroes n int32 words at p (a fill kernel, so that it can be captured).
hipError_t launch_zero_i32(int32_t* p, size_t n, hipStream_t stream);

}  // namespace gkv
