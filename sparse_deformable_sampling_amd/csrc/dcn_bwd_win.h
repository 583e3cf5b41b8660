// Configuration of the windowed backward kernel (internal header).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dcn_launch.h"

namespace dcn {

struct BwdWinCfg {
    int lq_log;       // log2 of the lanes per item
    int nv;           // 4 * nv channels per lane
    int ip;           // items per pass (threads / lanes per item)
    int tr;           // output rows per step
    int hy;           // halo rows above and below a step's footprint kept in the window
    int aw;           // window rows: (tr-1)*stride_h + (kernel_h-1)*dil_h + 2*hy + 3
    int chunk_rows;   // output rows per workgroup
    int chunks;       // row chunks per (image, group)
    int nwg;          // workgroups
    int threads;      // threads per workgroup
    int lds_bytes;    // aw * w * d * 8
    uint32_t x_bytes; // bytes of x (buffer extent)
};

// Fill `bc` for geometry G and storage type dtype; false if the windowed
// kernel does not apply.
bool plan_bwd_win(const Geom& G, int dtype, const void* x, const void* gout, int lds_limit, int num_cus,
                  BwdWinCfg* bc);

// x, off, mask, gout, goff and gmask in the storage type; gx is fp32.
hipError_t launch_dcn_backward_win(const Geom& G, const BwdWinCfg& bc, int dtype, const void* x, const void* off,
                                   const void* mask, const void* gout, float* gx, void* goff, void* gmask,
                                   hipStream_t s);

}  // namespace dcn
