// Configuration of the LDS sliding-window forward kernel (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcn_launch.h"

namespace dcn {

struct RingCfg {
    int pb;           // bytes of one pixel in LDS (all channels)
    int pitch;        // bytes of one ring row: (w + 2) pixels (zero column each side) + 16 bytes of bank skew
    int R;            // ring rows (plus one mirror slot)
    int nw;           // window rows a step may read
    int hy;           // halo rows above and below the footprint
    int tr;           // output rows per step
    int chunk_rows;   // output rows per workgroup
    int chunks;       // workgroups per image
    int nwg;          // workgroups
    int threads;      // threads per workgroup (one item per thread per step)
    int ring_bytes;   // (R + 1) * pitch: slot R mirrors slot 0
    int lds_bytes;    // ring + staging of one step's offsets and mask
    uint32_t x_bytes, off_bytes, mask_bytes;
};

// Fill `rc` for geometry G; false if the sliding-window kernel does not apply.
bool plan_ring(const Geom& G, int dtype, const void* x, const void* off, const void* mask, const void* out,
               int lds_limit, int num_cus, RingCfg* rc);

hipError_t launch_dcn_forward_ring(const Geom& G, const RingCfg& rc, int dtype, const void* x, const void* off,
                                   const void* mask, void* out, hipStream_t s);

// Per-device properties cached on first use (LDS bytes per workgroup, CU count).
void device_limits(int* lds_limit, int* num_cus);

}  // namespace dcn
