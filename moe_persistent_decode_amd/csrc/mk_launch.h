// mk_launch.h - host entry points into the device code (defined in mk_device.hip).
#pragma once
#include <hip/hip_runtime.h>

#include "mk_internal.h"

hipError_t mk_launch_interp(const mk_params& P, int head_dim, int grid, bool cooperative, hipStream_t stream);
hipError_t mk_launch_repack(const uint16_t* src, uint16_t* dst, int K, int N, int ld, int dst0, int dstep,
                            int nz, size_t src_zstride, size_t dst_zstride, hipStream_t stream);
// FP8 feed-forward weights: canonical [K x N] codes into chunk-pair panels
// (source panel j to dst0 + j * dstep, nz matrices), [E][F][H] down codes into
// per-slice column runs, and the three [E][F] scale vectors into
// (gate, up, down, 0) float4s.
hipError_t mk_launch_repack_fp8_panels(const uint8_t* src, uint8_t* dst, int K, int N, int dst0, int dstep, int nz,
                                       size_t src_zstride, size_t dst_zstride, hipStream_t stream);
hipError_t mk_launch_repack_fp8_d(const uint8_t* wd, uint8_t* dst, int F, int H, int E, hipStream_t stream);
hipError_t mk_launch_pack_scales(const float* sg, const float* su, const float* sd, float* dst, int n,
                                 hipStream_t stream);
hipError_t mk_interp_occupancy(int head_dim, int* blocks_per_cu);
// Device address of the static scratch array on `device` (looked up once per
// device, then cached), and a fill kernel zeroing n words.
hipError_t mk_static_scratch(int device, void** ptr);
hipError_t mk_launch_zero(uint32_t* p, int n, hipStream_t stream);
hipError_t mk_launch_fill(uint32_t* p, int n, uint32_t lo, uint32_t hi, hipStream_t stream);
hipError_t mk_launch_stream_read(const void* p, size_t n16, hipStream_t stream);
hipError_t mk_launch_litmus(uint32_t* msg, uint32_t* flag, uint32_t* ack, uint32_t* result, int pairs, int rounds,
                            int coherent, int64_t limit, hipStream_t stream);
