// Launchers of the pipelined kernel: declared for the host unit, defined and
// explicitly instantiated by gemm_unit.hip, compiled once per unit number of variants.inc.
#pragma once

#include <hip/hip_runtime.h>

#include "gemm_kernels.hpp"

namespace spg {

typedef void (*launch_fn)(const KArgs&, dim3, hipStream_t);

template <bool BF16, bool B_NK, int BM, int BN, int BK, int WM, int WN, int S, bool SWZ, int LDM,
          int PF, int SCHED, bool PERS, int MI>
void launch_pipelined(const KArgs& a, dim3 grid, hipStream_t st);

#ifdef SPG_DEFINE_LAUNCHERS
template <bool BF16, bool B_NK, int BM, int BN, int BK, int WM, int WN, int S, bool SWZ, int LDM,
          int PF, int SCHED, bool PERS, int MI>
void launch_pipelined(const KArgs& a, dim3 grid, hipStream_t st) {
    using G = Geom<BM, BN, BK, WM, WN, S>;
    if constexpr (LDM == 3) {
        // a producer wave and consumer waves (wave-specialized ring)
        using W = WsGeom<BF16, B_NK, BM, BN, BK, WM, WN, S>;
        hipLaunchKernelGGL((ws_gemm<BF16, B_NK, BM, BN, BK, WM, WN, S>), grid, dim3(W::NT), 0, st, a);
    } else if constexpr (PERS) {
        // the host sets a.persistent (and a grid of at most one workgroup per CU) only
        // for shapes the persistent kernel takes; otherwise the same tile, one per workgroup
        if (a.persistent)
            hipLaunchKernelGGL((pipelined_gemm<BF16, B_NK, BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, true, MI>),
                               grid, dim3(G::NT), 0, st, a);
        else
            hipLaunchKernelGGL((pipelined_gemm<BF16, B_NK, BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, false, MI>),
                               grid, dim3(G::NT), 0, st, a);
    } else {
        hipLaunchKernelGGL((pipelined_gemm<BF16, B_NK, BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, false, MI>),
                           grid, dim3(G::NT), 0, st, a);
    }
}
#endif

}  // namespace spg

#define SPG_INSTANTIATE_ALL(BM, BN, BK, WM, WN, S, SWZ, LDM, PF, SCHED, PERS, MI)                              \
    template void spg::launch_pipelined<false, false, BM, BN, BK, WM, WN, S, (SWZ != 0), LDM, PF, SCHED, (PERS != 0), MI>( \
        const spg::KArgs&, dim3, hipStream_t);                                                     \
    template void spg::launch_pipelined<false, true, BM, BN, BK, WM, WN, S, (SWZ != 0), LDM, PF, SCHED, (PERS != 0), MI>(  \
        const spg::KArgs&, dim3, hipStream_t);                                                     \
    template void spg::launch_pipelined<true, false, BM, BN, BK, WM, WN, S, (SWZ != 0), LDM, PF, SCHED, (PERS != 0), MI>(  \
        const spg::KArgs&, dim3, hipStream_t);                                                     \
    template void spg::launch_pipelined<true, true, BM, BN, BK, WM, WN, S, (SWZ != 0), LDM, PF, SCHED, (PERS != 0), MI>(   \
        const spg::KArgs&, dim3, hipStream_t);
