// Configuration of the LDS sliding-window forward kernel (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcn_launch.h"

namespace dcn {

struct RingCfg {
    int gs;           // channel groups per workgroup (a divisor of the group count)
    int gsets;        // group sets per image (= groups / gs)
    int pb;           // bytes of one pixel in LDS (gs groups)
    int cpp;          // 16-byte chunks per LDS pixel (pb / 16)
    int pitch;        // bytes of one ring row: (w + 3) pixels (two zero columns left, one right) + 80 bytes of bank skew
    int R;            // ring rows (slot R, one more, mirrors slot 0)
    int nw;           // window rows a step may read through LDS
    int hy;           // halo rows above and below the footprint
    int tr;           // output rows per step
    int chunk_rows;   // output rows per workgroup
    int chunks;       // row chunks per (image, group set)
    int nwg;          // workgroups
    int threads;      // threads per workgroup (one item per thread per step)
    int wmax;         // kernel variant: 16 (<= 128 VGPRs, four waves per SIMD) or 8 (<= 256 VGPRs)
    int row_iters;    // 1 KB copy instructions per wave for one input row
    int ring_bytes;   // (R + 1) * pitch
    int lds_bytes;    // the ring (each lane loads its offsets and mask into registers)
    uint32_t x_bytes, off_bytes, mask_bytes;   // buffer extents, rounded up to whole dwords
    int split_log;    // log2 of the lane items per channel group: a wide group (more than 32 bytes
                      // per pixel) runs as 2^split_log groups of its channels sharing its offsets and mask
};

// Fill `rc` for geometry G, and `gk` with the geometry the kernel runs on (G,
// or G with each wide group split into narrower ones); false if the
// sliding-window kernel does not apply.
bool plan_ring(const Geom& G, int dtype, const void* x, const void* off, const void* mask, const void* out,
               int lds_limit, int num_cus, RingCfg* rc, Geom* gk);

hipError_t launch_dcn_forward_ring(const Geom& G, const RingCfg& rc, int dtype, const void* x, const void* off,
                                   const void* mask, void* out, hipStream_t s);

// Per-device properties cached on first use (LDS bytes per workgroup, CU count).
void device_limits(int* lds_limit, int* num_cus);

}  // namespace dcn
