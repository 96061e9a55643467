// Host-side launch entry points of the kernels (internal to libsmla.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "smla_decode.hpp"

namespace smla {

// `map` places layer row `slot` in the allocation (identity for a layer-major pool).
hipError_t launch_pack(const void* src, const int32_t* slots, int32_t n, void* pool,
                       int64_t pool_rows, const RowMap& map, hipStream_t s);
hipError_t launch_unpack(const void* pool, int64_t pool_rows, const int32_t* rows, int32_t n,
                         void* out, hipStream_t s);
hipError_t launch_fp8_pack(const void* src, const int32_t* slots, int32_t n, void* pool, int64_t pool_rows,
                           hipStream_t s);
hipError_t launch_stage_fp8(const void* pool, int64_t pool_rows, const int32_t* idx,
                            int64_t entries, void* staged, hipStream_t s);
// Decode workgroups resident per CU for the kernel variant of this shape (LDS budget).
int decode_wgs_per_cu(bool fp8rows, int32_t NG, int variant);
// NVFP4 decode: 64-head blocks use the role-specialised kernel (decode_ws.hip), 32-head
// blocks the LDS-ring kernel; 16-head blocks the register-gather kernel (decode_regs.hip,
// variant 1), the LDS-ring kernel (variant 0) or the role-specialised kernel (variant 2).
hipError_t launch_decode_nvfp4(const DecodeArgs& a, hipStream_t s, int variant);
hipError_t launch_decode_nvfp4_regs(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_nvfp4_ws(const DecodeArgs& a, hipStream_t s, int heads, bool grouped);
// Grouped decode: the role-specialised kernel on union lists of token groups.
hipError_t launch_decode_grouped(const DecodeArgs& a, hipStream_t s);
// Union lists of token groups (group.hip).
hipError_t launch_group_union(const int32_t* idx, int32_t T, int32_t topk, int32_t tpg, int64_t pool_rows,
                              int32_t U, int32_t* uni, int32_t* count, hipStream_t s);
// Decode over FP8 rows (staged rows or an FP8 pool): 64-head blocks use the
// role-specialised kernel, 32- and 16-head blocks the LDS-ring kernel.
hipError_t launch_decode_fp8rows(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_fp8_ws(const DecodeArgs& a, hipStream_t s);
// Copies n segments of seg_bytes (a multiple of 16) from src segment src_ids[i] to dst
// segment dst_ids[i] (layout.hip); a null id array means segment i.
hipError_t launch_copy_segments(const void* src, int64_t src_segs, const int32_t* src_ids, void* dst,
                                int64_t dst_segs, const int32_t* dst_ids, int32_t n, int64_t seg_bytes,
                                hipStream_t s);
hipError_t launch_combine(const float* part_o, const float* part_lse, int32_t T, int32_t S,
                          int32_t H, void* out, float* lse, hipStream_t s);

}  // namespace smla
